// chunk.hip -- fused chunkwise KDA prefill for gfx950 (MI355X).
//
// Algebra: "Kimi Unveils Delta Attention and K3 Architecture Updates",
// section 6 (Chunkwise KDA), in the key-by-value orientation (S is d_k x d_v,
// decay multiplies key rows).  For one chunk of C = 64 tokens with incoming
// state S_c, let Gamma_i = prod_{m<=i} alpha_m (chunk-local cumulative decay,
// section 6.1/6.6 -- kept as a running product instead of exp of a prefix
// sum) and Gamma_L the decay over the whole chunk.  Then (section 6.3)
// R = Diag(beta) strict_tril(K_i Gamma_i / Gamma_j K_j^T) holds rho_ij =
// beta_i <k_j, D_{j+1:i} k_i>, (section 6.5) Aqk = tril(s Q_i Gamma_i /
// Gamma_j K_j^T) holds chi_ij, the provisional errors of section 6.2 are
// Ebar = Diag(beta) (V - (K Gamma) S_c), and the resolved errors are
// E = (I + R)^{-1} Ebar (the causal triangular solve of section 6.3).  beta
// scales whole rows, so it is applied to the R tiles and to Y rather than to
// the stored operands.  Finally (6.4, 6.5)
//
//   O_c     = (s Q Gamma) S_c + Aqk E
//   S_{c+1} = Diag(Gamma_L) S_c + K_end^T E,   K_end_i = k_i Gamma_L / Gamma_i.
//
// Decay references (KDA, one gate per key channel): every per-token factor
// is taken relative to the start of its token's 16-token block b, Pi_i =
// Gamma_i / Gamma_{16b-1}, and the chunk's stored operands are
//
//   QG_i = s q_i Pi_i      KG_i = k_i Pi_i      KI_i = k_i / Pi_i
//   K_end_i = k_i TQ_b / Pi_i           (TQ_b = T_b T_{b+1} .. T_3)
//
// with T_b the decay over block b.  The rest of each ratio is a product over
// whole blocks, per key channel: a tile across blocks I > J takes F_IJ =
// T_J .. T_{I-1} on its KI fragments, and block I's state products take P_I =
// T_0 .. T_{I-1} on the rows of S.  Inside one block Pi stays within
// [T_b, 1], so the operands stay in range however much the chunk decays as a
// whole; only a block decaying below 2^-120 in some channel (log alpha
// averaging below about -5.2 over 16 tokens) is beyond this, and that chunk
// runs the recurrence token by token on the same on-chip state instead.
//
// Design (one workgroup per (sequence, head) chain, all of d_v; 8 waves -- two
// per SIMD -- for d_v = 128, 4 for d_v = 64):
//  * the fp32 state never leaves the chip: each wave keeps its d_v/NW value
//    columns of S in registers for the whole sequence, and only the chunk's
//    S-independent operands are shared through LDS;
//  * S and E are consumed straight from the accumulator layout: two stacked
//    16-row accumulator tiles are one 32-deep MFMA operand once the k index is
//    relabelled (k = 4g + e for e < 4, 16 + 4g + e - 4 for e >= 4, g = lane/16);
//    every other operand is read from LDS in that same k order;
//  * operands contracted over tokens are stored row-major and read with
//    ds_read_b64_tr_b16 (gfx950 LDS transpose read);
//  * the triangular solve runs by 16-token blocks: the four 16x16 diagonal
//    blocks of I + R are inverted by forward substitution (S-independent, once
//    per chunk), then X_I = T_II (Y_I - sum_{J<I} R_IJ X_J) on MFMA;
//  * signs are folded into the stored operands (-V, -KI, hence -R and -Aqk)
//    so that the solve yields -E directly and no extra negation is needed;
//  * the next chunk's inputs are loaded into registers while this chunk is
//    computed, in three batches spread over the phases.
#include <stdlib.h>

#include "common.h"

namespace kda {

// ============================================================ lane shifts
// DPP moves (a lane reads a neighbour's register inside one VALU instruction,
// with no LDS traffic); lanes without a valid source get 1.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), CTRL,
                                                    ROW_MASK, 0xf, false));
}
// x of lane l - D inside the lane's 16-lane row (1 for the first D lanes)
template <int D>
__device__ __forceinline__ float dpp_row_shr(float x) { return dpp1<0x110 + D, 0xf>(x); }
// x of lane l - D inside the lane's 16-lane row, 0 for the first D lanes (the
// zero fill lets the compiler fuse the move into the consuming add)
template <int D>
__device__ __forceinline__ float dpp_row_shr0(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + D, 0xf, 0xf, true));
}

// ============================================================ operand policies
typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// The lane id, re-materialised wherever it is asked for: the volatile asm keeps
// the compiler from hoisting lane-dependent addresses and constants out of the
// chunk loop, where they would occupy registers for the whole kernel.  Each
// phase asks once and passes it down.
__device__ __forceinline__ int lane_fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// No instruction may be scheduled across this point (nothing is emitted).
// Used to bound how far the scheduler hoists loads, which otherwise keeps far
// more values live than there are registers.
__device__ __forceinline__ void compiler_fence() { __builtin_amdgcn_sched_barrier(0); }

// All LDS addressing is done on address_space(3) pointers (32-bit), so that
// constant offsets fold into the ds_* instructions' immediate field.
#define LDS __attribute__((address_space(3)))

template <class P, class Q>
__device__ __forceinline__ LDS P* lds_ptr(LDS Q* p) {
  return (LDS P*)(p);
}

// ------------------------------------------------------------ buffer access
// Raw buffer loads/stores with a workgroup-uniform resource: the base lives in
// SGPRs, each lane supplies a 32-bit byte offset, and any access at or beyond
// num_records bytes reads as zero (loads) or is dropped (stores).  That is
// how a chunk's padding tokens come out as zeros without branches.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define KDA_BUF_FLAGS 0x00020000

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           KDA_BUF_FLAGS);
}
template <class V> __device__ __forceinline__ V buf_load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0);
template <> __device__ __forceinline__ uint16_t buf_load<uint16_t>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
}
template <> __device__ __forceinline__ uint32_t buf_load<uint32_t>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
}
template <> __device__ __forceinline__ float buf_load<float>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0));
}
template <> __device__ __forceinline__ u32x2 buf_load<u32x2>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
template <> __device__ __forceinline__ f32x2 buf_load<f32x2>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0));
}
template <> __device__ __forceinline__ f32x4 buf_load<f32x4>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
template <> __device__ __forceinline__ u32x4 buf_load<u32x4>(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, off, 0, 0);
}

// The k order of a 32-deep operand fragment: inside every block of 32
// indices, position 8g + e holds index 4g + e and position 8g + 4 + e holds
// index 16 + 4g + e (g, e < 4).  Lane group g of a fragment over k0 .. k0+31
// holds exactly the indices at positions k0 + 8g .. k0 + 8g + 7, and any four
// consecutive indices starting at a multiple of 4 stay contiguous.
__device__ __forceinline__ int frag_pos(int c) {
  const int r = c & 31;
  return (c & ~31) + 8 * ((r & 15) >> 2) + ((r & 16) >> 2) + (r & 3);
}

// bf16 operands, fp32 accumulation: v_mfma_f32_16x16x32_bf16 / 16x16x16_bf16.
struct OpBf16 {
  typedef uint16_t T;
  static constexpr int PAD_RM = 8;    // row padding (elements) of buffers read as 8-byte rows
  // Row padding of buffers read as 16-byte rows by 16 consecutive rows: a row
  // stride of 8 (mod 16) dwords puts the 32 lanes of each half-wave on 32
  // distinct 8-byte bank pairs in both passes of ds_read_b128.
  static constexpr int PAD_B128 = 16;
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
  static __device__ __forceinline__ F16 ld16_rm(int l, const LDS T* X, int ld, int row0, int k0) {
    return *lds_ptr<const F16>(X + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
  }
  // X row-major: lane gets X[k0 + 4g + e][m0 + l%16] (transpose read)
  static __device__ __forceinline__ F16 ld16_tr(int l, const LDS T* X, int ld, int k0, int m0) {
    const int j = l & 15;
    const LDS T* p = X + (k0 + 4 * (l >> 4) + (j >> 2)) * ld + m0 + 4 * (j & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(p));
  }
  static __device__ __forceinline__ F32 ld32_rm(int l, const LDS T* X, int ld, int row0, int k0) {
    return F32{ld16_rm(l, X, ld, row0, k0), ld16_rm(l, X, ld, row0, k0 + 16)};
  }
  static __device__ __forceinline__ F32 ld32_tr(int l, const LDS T* X, int ld, int k0, int m0) {
    return F32{ld16_tr(l, X, ld, k0, m0), ld16_tr(l, X, ld, k0 + 16, m0)};
  }
  // Permuted buffers (the operands over key channels, the key-major -K_end
  // over tokens) are stored in fragment order (frag_pos), so that one 16-byte
  // read gives a lane both halves of its fragment.
  static constexpr bool PERMUTED = true;
  static __device__ __forceinline__ int perm_pos(int c) { return frag_pos(c); }
  static __device__ __forceinline__ F32 ld32_rmp(int l, const LDS T* X, int ld, int row0, int k0) {
    const i16x8 v = *lds_ptr<const i16x8>(X + (row0 + (l & 15)) * ld + k0 + 8 * (l >> 4));
    return F32{__builtin_shufflevector(v, v, 0, 1, 2, 3), __builtin_shufflevector(v, v, 4, 5, 6, 7)};
  }
  // transpose read of a permuted buffer: lane gets X[k0 + 4g + e][channel
  // c0 + l%16] with c0 = a multiple of 16 (position base m0 = perm_pos(c0))
  static __device__ __forceinline__ F16 ld16_trp(int l, const LDS T* X, int ld, int k0, int m0) {
    const int j = l & 15;
    const LDS T* p = X + (k0 + 4 * (l >> 4) + (j >> 2)) * ld + m0 + 8 * (j & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(p));
  }
  static __device__ __forceinline__ F32 ld32_trp(int l, const LDS T* X, int ld, int k0, int m0) {
    return F32{ld16_trp(l, X, ld, k0, m0), ld16_trp(l, X, ld, k0 + 16, m0)};
  }
  // write accumulator tile t (rows row0 + 4g + r, column col0 + l%16) transposed:
  // Xt[col0 + l%16][row0 + 4g + r] for r = 0..3 (four contiguous elements)
  static __device__ __forceinline__ void st_ct(int l, LDS T* Xt, int ld, int col0, int row0, f32x4 t) {
    *lds_ptr<F16>(Xt + (col0 + (l & 15)) * ld + row0 + 4 * (l >> 4)) = pack(t);
  }
};

// fp32 operands: v_mfma_f32_16x16x4_f32, four (or eight) per fragment.
struct OpF32 {
  typedef float T;
  static constexpr int PAD_RM = 4;
  static constexpr int PAD_B128 = 4;   // (8 would avoid the conflicts but not fit in LDS)
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
  static __device__ __forceinline__ F16 ld16_rm(int l, const LDS T* X, int ld, int row0, int k0) {
    return *lds_ptr<const F16>(X + (row0 + (l & 15)) * ld + k0 + 4 * (l >> 4));
  }
  static __device__ __forceinline__ F16 ld16_tr(int l, const LDS T* X, int ld, int k0, int m0) {
    const LDS T* p = X + (k0 + 4 * (l >> 4)) * ld + m0 + (l & 15);
    F16 r;
    r[0] = *lds_ptr<const T>(p);
    r[1] = *lds_ptr<const T>(p + ld);
    r[2] = *lds_ptr<const T>(p + 2 * ld);
    r[3] = *lds_ptr<const T>(p + 3 * ld);
    return r;
  }
  static __device__ __forceinline__ F32 ld32_rm(int l, const LDS T* X, int ld, int row0, int k0) {
    return F32{ld16_rm(l, X, ld, row0, k0), ld16_rm(l, X, ld, row0, k0 + 16)};
  }
  static __device__ __forceinline__ F32 ld32_tr(int l, const LDS T* X, int ld, int k0, int m0) {
    return F32{ld16_tr(l, X, ld, k0, m0), ld16_tr(l, X, ld, k0 + 16, m0)};
  }
  static __device__ __forceinline__ void st_ct(int l, LDS T* Xt, int ld, int col0, int row0, f32x4 t) {
    *lds_ptr<F16>(Xt + (col0 + (l & 15)) * ld + row0 + 4 * (l >> 4)) = t;
  }
  // fp32 operands keep the natural channel order
  static constexpr bool PERMUTED = false;
  static __device__ __forceinline__ int perm_pos(int c) { return c; }
  static __device__ __forceinline__ F32 ld32_rmp(int l, const LDS T* X, int ld, int row0, int k0) {
    return ld32_rm(l, X, ld, row0, k0);
  }
  static __device__ __forceinline__ F32 ld32_trp(int l, const LDS T* X, int ld, int k0, int m0) {
    return ld32_tr(l, X, ld, k0, m0);
  }
};

// ============================================================ raw input words
// BYTES of consecutive input kept as raw dwords, so that a prefetch stays in
// flight until the next chunk unpacks it.  Loaded as 16-byte pieces (plus one
// 8-byte piece when BYTES is not a multiple of 16).
template <int BYTES>
struct RawWords {
  static_assert(BYTES % 8 == 0, "raw vectors are whole 8-byte pieces");
  static constexpr int N16 = BYTES / 16, N8 = (BYTES % 16) / 8;
  u32x4 q[N16 > 0 ? N16 : 1];
  u32x2 d;
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
#pragma unroll
    for (int i = 0; i < N16; ++i) q[i] = buf_load<u32x4>(r, voff + 16 * i, soff);
    if (N8) d = buf_load<u32x2>(r, voff + 16 * N16, soff);
  }
  __device__ __forceinline__ uint32_t word(int i) const {
    return i < 4 * N16 ? q[i / 4][i % 4] : d[i - 4 * N16];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < (N16 > 0 ? N16 : 1); ++i) q[i] = u32x4{0u, 0u, 0u, 0u};
    d = u32x2{0u, 0u};
  }
};

// N elements of I/O type Io as floats
template <class Io, int N>
struct RawIo {
  RawWords<N * (int)sizeof(typename Io::storage)> w;
  __device__ __forceinline__ void unpack(float* o) const {
#pragma unroll
    for (int e = 0; e < N; ++e) {
      if (Io::is_bf16) {
        const uint32_t x = w.word(e / 2);
        o[e] = __uint_as_float((e & 1) ? (x & 0xffff0000u) : (x << 16));
      } else {
        o[e] = __uint_as_float(w.word(e));
      }
    }
  }
};

// ============================================================ configuration
// Four waves per workgroup; wave w owns value columns [w d_v/4, (w+1) d_v/4)
// of the state for the whole sequence.
template <int DK_, int DV_, class Io_, class Op_, int NW_ = 4, bool SG_ = false, bool FU_ = false>
struct ChunkCfg {
  static constexpr int DK = DK_, DV = DV_;
  // SG: one gate per (token, head) shared by every key channel (Gated
  // DeltaNet); otherwise one per key channel (KDA)
  static constexpr bool SG = SG_;
  // FU: the raw inputs pass through the transforms of a Prologue (common.h)
  static constexpr bool FU = FU_;
  typedef Io_ Io;
  typedef Op_ Op;
  typedef typename Op::T T;
  static constexpr int C = 64;          // tokens per chunk
  static constexpr int NB = 4;          // 16-token blocks per chunk
  static constexpr int NW = NW_;        // waves per workgroup (4 or 8)
  static constexpr int NTHREADS = 64 * NW;
  static constexpr int NKS = DK / 32;   // 32-deep steps over key channels
  static constexpr int MTK = DK / 16;   // 16-row tiles over key channels
  static constexpr int VW = DV / NW;    // value columns per wave
  static constexpr int NVT = VW / 16;   // 16-column value tiles per wave
  // prep layout: each lane holds 8 consecutive key channels of TPL tokens
  static constexpr int CPL = 8;
  static constexpr int CQ = DK / NW / CPL;   // lanes across a wave's key channels
  static constexpr int TG = 64 / CQ;         // token groups
  static constexpr int TPL = C / TG;         // tokens per lane
  static constexpr int VPL = VW / CQ;        // value channels per lane
  static_assert((NW == 4 || NW == 8) && CQ * TG == 64 && TPL * TG == C && VPL * CQ == VW,
                "layout");
  // LDS leading dimensions (elements)
  // Row strides are chosen against LDS bank conflicts (gfx950: 64 dword banks per
  // half-wave for 8-byte reads, ds_read_b128 in two 8-byte passes): buffers read
  // as 16-byte row fragments take PAD_B128, the others PAD_RM.
  static constexpr int LD_K = DK + Op::PAD_B128;  // QG, KG, KIn [C][LD_K]
  static constexpr int LD_V = DV + Op::PAD_RM;    // -V (buffer BV) [C][LD_V]
  static constexpr int LD_RR = C + Op::PAD_RM;    // RR [C][LD_RR] (8-byte row reads)
  static constexpr int LD_AQ = C + Op::PAD_B128;  // AQ [C][LD_AQ] (16-byte row reads)
  static constexpr int SZ = sizeof(T);
  // LDS byte offsets.
  static constexpr int OFF_QG = 0;
  static constexpr int OFF_KG = OFF_QG + C * LD_K * SZ;
  static constexpr int OFF_KI = OFF_KG + C * LD_K * SZ;
  static constexpr int OFF_RD = OFF_KI + C * LD_K * SZ;
  static constexpr int RD_LD = 20;     // floats per column of a diagonal block (padded)
  static constexpr int LD_OS = DV + Op::PAD_RM;  // OST [C][LD_OS]
  static constexpr int OFF_OS = OFF_RD + NB * 16 * RD_LD * 4;
  static constexpr int OFF_BV = OFF_OS + C * LD_OS * SZ;
  static constexpr int OFF_AQ = OFF_BV + C * LD_V * SZ;
  static constexpr int OFF_RT = OFF_AQ + C * LD_AQ * SZ;
  static constexpr int OFF_TD = OFF_RT + C * LD_RR * SZ;
  static constexpr int LD_KT = C + Op::PAD_B128;  // KIT [DK][LD_KT]
  static constexpr int OFF_KT = OFF_TD + NB * 16 * 16 * SZ;
  // KDA decay factors per key channel, fp32 in fragment order (frag_pos).
  // Each wave's own channels, read back only by that wave: [4][DK] the block
  // totals T_b, and per block the factors that take the block-local decay
  // to the operands' reference (FA) and -k / (that reference) to -K_end (FM).
  // For the tiles and scan_y: [4][DK] the state factors of block-referenced
  // channels (P_b = T_0 .. T_{b-1}, else 1), [6][DK] their tile factors
  // F_IJ = T_J .. T_{I-1} (else 1) of the pairs I > J in the order (1,0)
  // (2,0) (2,1) (3,0) (3,1) (3,2), and a mask of the chunk-referenced
  // channels.
  static constexpr int OFF_DT = OFF_KT + DK * LD_KT * SZ;
  static constexpr int OFF_FA = OFF_DT + 4 * DK * 4;
  static constexpr int OFF_FM = OFF_FA + 4 * DK * 4;
  static constexpr int OFF_DP = OFF_FM + 4 * DK * 4;
  static constexpr int OFF_DF = OFF_DP + 4 * DK * 4;
  // [DK] uint16: 0xffff for chunk-referenced channels, 0 for block-referenced
  static constexpr int OFF_MK = OFF_DF + 6 * DK * 4;
  static constexpr int SZ_D = SG ? 0 : OFF_MK - OFF_DT + ((DK * 2 + 15) / 16) * 16;
  static constexpr int OFF_GL = OFF_DT + SZ_D;
  static_assert(SG || OFF_GL >= OFF_MK + DK * 2, "the decay factors fit their region");
  static constexpr int OFF_BT = OFF_GL + DK * 4;          // beta of the chunk's tokens
  static constexpr int OFF_FL = OFF_BT + C * 4;
  // FU only: per-wave partial squared norms of q and k, [C][NW] each, and the
  // head's gate biases [DK]
  static constexpr int OFF_NM = OFF_FL + 64;
  static constexpr int SZ_NM = FU ? 2 * C * NW * 4 + DK * 4 : 0;
  // SG only: per-token factors of the raw operands, C floats each (SV_*), and
  // the log2 decay of each 16-token block (4 floats)
  static constexpr int OFF_SV = OFF_NM + SZ_NM;
  static constexpr int SZ_SV = SG ? (7 * C + 4) * 4 : 0;
  static constexpr int LDS_TOTAL = OFF_SV + SZ_SV;
  static_assert(LDS_TOTAL <= 160 * 1024, "LDS budget");
  static_assert(LDS_TOTAL >= (KDA_LPT_MAX + 1) * 4, "LDS holds the length ranking");
  static_assert(OFF_KG % 16 == 0 && OFF_KI % 16 == 0 && OFF_RD % 16 == 0 && OFF_OS % 16 == 0 && OFF_FL % 16 == 0 &&
                OFF_BV % 16 == 0 && OFF_AQ % 16 == 0 && OFF_RT % 16 == 0 && OFF_TD % 16 == 0 &&
                OFF_GL % 16 == 0 && OFF_BT % 16 == 0 && OFF_KT % 16 == 0 && OFF_DT % 16 == 0 && (LD_K * SZ) % 16 == 0 &&
                (LD_KT * SZ) % 16 == 0 && (LD_V * SZ) % 16 == 0 && (LD_AQ * SZ) % 16 == 0 &&
                (LD_RR * SZ) % 8 == 0 && (LD_OS * SZ) % 16 == 0, "LDS alignment");
};

// log2 of the threshold below which a 16-token block's decay T_b makes
// k / Pi unsafe (Pi >= T_b inside the block, so 1 / Pi stays below 2^120).
// With the gate transform, log alpha >= -5 per token keeps every block above
// 2^-115.5.
#define KDA_BLOCK_LOG2_MIN (-120.f)
// log2 of the block decay down to which chunk-start references stay in use
// (four blocks then decay by at most 2^-100)
#define KDA_CHUNK_REF_LOG2_MIN (-25.f)
// log2 of the bound below which the state factors of a block-referenced
// channel (P_b for b >= 1, all at most T_0) are taken as 0: the operands they
// multiply are bounded by |k| and |s q| (Pi <= 1), so the terms stay below
// 2^-40 of |k| |S|, far under fp32 rounding of the sums they enter.  (The
// tile factors F_IJ are always applied: the -k / Pi_j they multiply grows as
// they shrink.)
#define KDA_STATE_LOG2_NEGLIGIBLE (-40.f)

// Reference modes of a chunk (wave-uniform after the flag vote): every key
// channel chunk-referenced; some block-referenced, all with negligible state
// factors (a channel mask replaces them in the state products); some with
// state factors that must be applied.
enum { KDA_MODE_CHUNK = 0, KDA_MODE_MASK = 1, KDA_MODE_SCALE = 2 };

// ============================================================ the kernel
template <class Cfg>
struct ChunkKernel {
  typedef typename Cfg::Io Io;
  typedef typename Cfg::Op Op;
  typedef typename Cfg::T T;
  static constexpr int DK = Cfg::DK, DV = Cfg::DV, C = Cfg::C, NW = Cfg::NW;
  static constexpr int CPL = Cfg::CPL, VPL = Cfg::VPL, CQ = Cfg::CQ, TG = Cfg::TG,
                       TPL = Cfg::TPL, VW = Cfg::VW;
  static constexpr int NKS = Cfg::NKS, MTK = Cfg::MTK, NWT = Cfg::NWT, NVT = Cfg::NVT;

  struct Raw {
    RawWords<CPL * 4> g[TPL];   // per-channel gates (KDA)
    float gs[TPL];              // the per-token gate (Gated DeltaNet)
    RawIo<Io, CPL> q[TPL], k[TPL];
    RawIo<Io, VPL> v[TPL];
    float beta;
  };
  enum { LOAD_Q = 1, LOAD_K = 2, LOAD_V = 4, LOAD_G = 8, LOAD_ALL = 15 };

  // N contiguous LDS elements written as one vector store
  template <int N>
  static __device__ __forceinline__ void st_vec(LDS T* p, const T (&x)[N]) {
    typedef T vec __attribute__((ext_vector_type(N)));
    vec v;
#pragma unroll
    for (int c = 0; c < N; ++c) v[c] = x[c];
    *lds_ptr<vec>(p) = v;
  }

  // ---------------------------------------------------------------- loads
  // Prep layout: wave w, lane l = tg * CQ + cq holds tokens TPL*tg + t
  // (t < TPL), key channels kc0 .. kc0+7 with kc0 = w*DK/4 + 8 cq, and value
  // channels vc0 .. vc0+VPL-1 with vc0 = w*DV/4 + VPL cq.  Offsets are
  // relative to the chunk's first token, hence the same for every chunk.
  struct Offsets {
    uint32_t qk, g, v, beta;   // lane byte offsets of its first token
    uint32_t sqk, sg, sv;      // byte strides between consecutive tokens
  };
  static __device__ __forceinline__ Offsets lane_offsets(int H) {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const int tg = l / CQ, cq = l % CQ;
    const int kc0 = w * (DK / NW) + CPL * cq;
    const int vc0 = w * VW + VPL * cq;
    constexpr uint32_t E = sizeof(typename Io::storage);
    Offsets o;
    o.sqk = (uint32_t)H * DK * E;
    o.sg = (uint32_t)H * (Cfg::SG ? 1 : DK) * 4;
    o.sv = (uint32_t)H * DV * E;
    o.qk = (uint32_t)(TPL * tg) * o.sqk + kc0 * E;
    o.g = (uint32_t)(TPL * tg) * o.sg + (Cfg::SG ? 0 : kc0 * 4);
    o.v = (uint32_t)(TPL * tg) * o.sv + vc0 * E;
    o.beta = (uint32_t)l * H * 4;
    return o;
  }
  // Loads of one chunk (first token row0, clen valid tokens); padding tokens
  // read as zeros through the resources' size limit.
  template <int PART>
  static __device__ __forceinline__ void load_raw(Raw& r, const Offsets& o, const void* q,
                                                  const void* k, const void* v, const float* g,
                                                  const float* beta, size_t row0, int H, int h,
                                                  int clen) {
    constexpr size_t E = sizeof(typename Io::storage);
    const size_t e0 = row0 * H + h;   // element row of the chunk's first token, this head
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)q + e0 * DK * E, clen * o.sqk);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const char*)k + e0 * DK * E, clen * o.sqk);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const char*)v + e0 * DV * E, clen * o.sv);
    const __amdgpu_buffer_rsrc_t rg =
        make_rsrc((const char*)g + e0 * (Cfg::SG ? 1 : DK) * 4, clen * o.sg);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(beta + e0, (uint32_t)clen * H * 4);
    // lane part in the VGPR offset, the token step in the scalar offset
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      if (PART & LOAD_Q) r.q[t].w.load(rq, o.qk, t * o.sqk);
      if (PART & LOAD_K) r.k[t].w.load(rk, o.qk, t * o.sqk);
      if (PART & LOAD_V) r.v[t].w.load(rv, o.v, t * o.sv);
      if (PART & LOAD_G) {
        if (Cfg::SG)
          r.gs[t] = buf_load<float>(rg, o.g, t * o.sg);
        else
          r.g[t].load(rg, o.g, t * o.sg);
      }
    }
    if (PART & LOAD_V) r.beta = buf_load<float>(rb, o.beta);   // lane l: beta of token l
  }

  // ---------------------------------------------------------------- norms (FU)
  // Per-wave partial squared norms of the chunk's raw q and k rows: the CQ
  // lanes that share a token add their channels, then one of them stores the
  // wave's partial to NQ / NK [token][wave].
  static __device__ __forceinline__ void norm_partials(const Raw& r, LDS char* smem) {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const int tg = l / CQ, cq = l % CQ;
    LDS float* NQ = (LDS float*)(smem + Cfg::OFF_NM);
    LDS float* NK = NQ + C * NW;
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      float qv[CPL], kv[CPL];
      r.q[t].unpack(qv);
      r.k[t].unpack(kv);
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        sq += qv[c] * qv[c];
        sk += kv[c] * kv[c];
      }
#pragma unroll
      for (int d = 1; d < CQ; d <<= 1) {
        sq += __shfl_xor(sq, d);
        sk += __shfl_xor(sk, d);
      }
      if (cq == 0) {
        NQ[(TPL * tg + t) * NW + w] = sq;
        NK[(TPL * tg + t) * NW + w] = sk;
      }
    }
  }

  // ---------------------------------------------------------------- raw operands (SG)
  // 8 consecutive channels of one row straight from the raw words (the I/O
  // type is the operand type), sign bits XOR-ed with `sign`.
  template <int NB>
  static __device__ __forceinline__ void st_raw8(LDS T* row, int c0, const RawWords<NB>& w,
                                                 uint32_t sign) {
    if constexpr (Op::PERMUTED) {
      *lds_ptr<u32x2>(row + Op::perm_pos(c0)) = u32x2{w.word(0) ^ sign, w.word(1) ^ sign};
      *lds_ptr<u32x2>(row + Op::perm_pos(c0 + 4)) = u32x2{w.word(2) ^ sign, w.word(3) ^ sign};
    } else {
      T y[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = __uint_as_float(w.word(c) ^ sign);
      st_chunk(row + c0, y);
    }
  }
  // Gated DeltaNet (one gate per token).  With a scalar decay the gate
  // factors of every product are per-token scalars, so the operands stay the
  // raw inputs: QG = q, KG = k, -KI = -k (and the key-major -k), -V, and the
  // scalars go to LDS, C floats each, for the epilogues of the products:
  //   SV_G   gamma_i: prefix sum of log2 alpha from the start of token i's
  //          16-token block (block-local, so differences of nearby tokens stay
  //          exact to rounding however much the chunk decayed before them)
  //   SV_RQ  rq_i = scale / |q_i|      SV_RK  rk_i = 1 / |k_i|  (1 without the
  //                                    L2-norm transform)
  //   SV_BK  beta_i rk_i               SV_FY  beta_i Gamma_i rk_i   (Y)
  //   SV_FO  Gamma_i rq_i   (O)        SV_FS  rk_i Gamma_L / Gamma_i (S update)
  //   SV_T   (4 floats) the total log2 decay of each 16-token block
  // Every factor is at most 1 in size (for log alpha <= 0): no decay is too
  // strong for this form, so there is no guard.  Each exponent is formed from
  // block-local sums and block totals, never as a difference of two prefix
  // sums over the whole chunk.
  enum { SV_G = 0, SV_RQ = 1, SV_RK = 2, SV_BK = 3, SV_FY = 4, SV_FO = 5, SV_FS = 6, SV_T = 7 };
  static __device__ __forceinline__ void prep_sg(const Raw& r, LDS char* smem, float scale,
                                                 const Prologue& pro, float ea, int hi) {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const int tg = l / CQ, cq = l % CQ;
    const int kc0 = w * (DK / NW) + CPL * cq;
    const int vc0 = w * VW + VPL * cq;
    LDS T* QG = (LDS T*)(smem + Cfg::OFF_QG);
    LDS T* KG = (LDS T*)(smem + Cfg::OFF_KG);
    LDS T* KI = (LDS T*)(smem + Cfg::OFF_KI);
    LDS T* BV = (LDS T*)(smem + Cfg::OFF_BV);
    LDS T* KIT = (LDS T*)(smem + Cfg::OFF_KT);
    LDS float* GL = (LDS float*)(smem + Cfg::OFF_GL);
    LDS float* BT = (LDS float*)(smem + Cfg::OFF_BT);
    LDS float* SV = (LDS float*)(smem + Cfg::OFF_SV);
    constexpr uint32_t SIGN = Cfg::SZ == 2 ? 0x80008000u : 0x80000000u;
    constexpr float LOG2E = 1.4426950408889634f;

    // gamma of the lane's tokens: a running sum over its TPL tokens, an
    // inclusive scan of the group sums over the lanes cq + CQ tg within each
    // 16-token block (segments of GPB groups), then one group back.  Rows
    // past hi keep log alpha = 0 under the gate transform (identity tokens).
    const bool xg = Cfg::FU && (pro.flags & PRO_GATE);
    const float gb = xg ? ((const LDS float*)(smem + Cfg::OFF_NM + 2 * C * NW * 4))[0] : 0.f;
    float gam[TPL];
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      const bool real = TPL * tg + t < hi;
      const float la = xg ? (real ? gate_logalpha(r.gs[t], ea, gb) : 0.f) : r.gs[t];
      gam[t] = (t == 0 ? 0.f : gam[t - 1]) + la * LOG2E;
    }
    constexpr int GPB = 16 / TPL;               // token groups per 16-token block
    static_assert(16 % TPL == 0, "a lane's tokens stay in one block");
    float x = gam[TPL - 1];
#pragma unroll
    for (int d = 1; d < GPB; d <<= 1) {
      const float y = __shfl_up(x, CQ * d);
      if (tg % GPB >= d) x += y;
    }
    float tb[4];                                // block totals, in every lane
#pragma unroll
    for (int b = 0; b < 4; ++b) tb[b] = __shfl(x, CQ * (GPB * b + GPB - 1));
    const float y = __shfl_up(x, CQ);
    const float e0 = (tg % GPB) ? y : 0.f;
#pragma unroll
    for (int t = 0; t < TPL; ++t) gam[t] += e0;  // block-local gamma
    const int blk = TPL * tg / 16;
    float before = 0.f, after = 0.f;            // the blocks before / after the lane's
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < blk) before += tb[b];
      if (b > blk) after += tb[b];
    }
    if (w == 0 && l < 4) SV[SV_T * C + l] = l == 0 ? tb[0] : l == 1 ? tb[1] : l == 2 ? tb[2] : tb[3];
    if (tg == 0) {
      const float gl = exp2f((tb[0] + tb[1]) + (tb[2] + tb[3]));
      *lds_ptr<f32x4>(GL + kc0) = f32x4{gl, gl, gl, gl};
      *lds_ptr<f32x4>(GL + kc0 + 4) = f32x4{gl, gl, gl, gl};
    }
    const float beta = (Cfg::FU && (pro.flags & PRO_BETA_SIGMOID)) ? sigmoid_f(r.beta) : r.beta;
    if (w == 0) BT[l] = beta;                   // lane l holds beta of token l

#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      const int i = TPL * tg + t;
      st_raw8(QG + i * Cfg::LD_K, kc0, r.q[t].w, 0u);
      st_raw8(KG + i * Cfg::LD_K, kc0, r.k[t].w, 0u);
      st_raw8(KI + i * Cfg::LD_K, kc0, r.k[t].w, SIGN);
      st_neg(BV + i * Cfg::LD_V + vc0, r.v[t]);
      if (w == 0) {
        float rq = scale, rk = 1.f;
        if (Cfg::FU && (pro.flags & PRO_L2NORM)) {
          // the token's squared norms: the sum of the waves' partials
          const LDS float* NQ = (const LDS float*)(smem + Cfg::OFF_NM) + i * NW;
          const LDS float* NK = NQ + C * NW;
          float sq = 0.f, sk = 0.f;
#pragma unroll
          for (int j = 0; j < NW; j += 4) {
            const f32x4 a = *lds_ptr<const f32x4>(NQ + j), b = *lds_ptr<const f32x4>(NK + j);
            sq += (a[0] + a[1]) + (a[2] + a[3]);
            sk += (b[0] + b[1]) + (b[2] + b[3]);
          }
          rq *= __builtin_amdgcn_rsqf(sq + PRO_NORM_EPS);
          rk = __builtin_amdgcn_rsqf(sk + PRO_NORM_EPS);
        }
        const float bi = __shfl(beta, i);
        if (cq == 0) {
          const float G = exp2f(before + gam[t]);
          SV[SV_G * C + i] = gam[t];
          SV[SV_RQ * C + i] = rq;
          SV[SV_RK * C + i] = rk;
          SV[SV_BK * C + i] = bi * rk;
          SV[SV_FY * C + i] = bi * G * rk;
          SV[SV_FO * C + i] = G * rq;
          SV[SV_FS * C + i] = exp2f((tb[blk] - gam[t]) + after) * rk;
        }
      }
    }
    // key-major -k: KIT[channel][token], the lane's TPL consecutive tokens
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      LDS T* p = KIT + (kc0 + c) * Cfg::LD_KT + Op::perm_pos(TPL * tg);
      if constexpr (Cfg::SZ == 2 && TPL == 2) {
        const uint32_t a = r.k[0].w.word(c >> 1), b = r.k[1].w.word(c >> 1);
        const uint32_t pr = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        *lds_ptr<uint32_t>(p) = pr ^ SIGN;
      } else {
        T kt[TPL];
#pragma unroll
        for (int t = 0; t < TPL; ++t) {
          float kv[CPL];
          r.k[t].unpack(kv);
          kt[t] = Op::cvt(-kv[c]);
        }
        st_vec(p, kt);
      }
    }
  }

  // ---------------------------------------------------------------- prep
  // Inclusive sum scan over the lanes of one cq inside a 16-lane DPP row
  // (stride CQ): the token groups of one 16-token block.
  template <int D>
  static __device__ __forceinline__ float row_scan(float x) {
    if constexpr (D < 16) {
      x += dpp_row_shr0<D>(x);
      return row_scan<2 * D>(x);
    } else {
      return x;
    }
  }

  // Lane-dependent LDS byte offsets of prep's accesses, formed once per chain
  // (they do not change from chunk to chunk), so that each access is a base
  // register plus an immediate offset.
  struct PrepAddr {
    int rowk;   // row TPL tg, key channel kc0 of a [C][LD_K] operand buffer
    int rowv;   // row TPL tg, value channel vc0 of the [C][LD_V] buffer
    int kit;    // key row kc0, token TPL tg of the key-major [DK][LD_KT] buffer
    int fac;    // block tg / GPB, key channel kc0 of a [4][DK] float factor array
  };
  static __device__ __forceinline__ PrepAddr prep_addr() {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const int tg = l / CQ, cq = l % CQ;
    const int kc0 = w * (DK / NW) + CPL * cq;
    const int vc0 = w * VW + VPL * cq;
    PrepAddr a;
    a.rowk = ((TPL * tg) * Cfg::LD_K + Op::perm_pos(kc0)) * Cfg::SZ;
    a.rowv = ((TPL * tg) * Cfg::LD_V + vc0) * Cfg::SZ;
    a.kit = (kc0 * Cfg::LD_KT + Op::perm_pos(TPL * tg)) * Cfg::SZ;
    a.fac = ((TPL * tg / 16) * DK + frag_pos(kc0)) * 4;
    return a;
  }
  // Channels c0 .. c0 + 7 of one operand row at p (the lane's position of c0):
  // in the permuted bf16 order c0 + 4 .. c0 + 7 sit 8 elements on, in the fp32
  // order 4.
  static __device__ __forceinline__ void st8_at(LDS T* p, const float (&x)[8]) {
    if constexpr (Op::PERMUTED) {
      *lds_ptr<u32x2>(p) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *lds_ptr<u32x2>(p + 8) = u32x2{pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    } else {
      *lds_ptr<f32x4>(p) = f32x4{x[0], x[1], x[2], x[3]};
      *lds_ptr<f32x4>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
  }

  // KDA: the decay factors and the gate-scaled operands of one chunk (tokens
  // [0, hi) real, the rest identity tokens), "Kimi Unveils Delta Attention
  // and K3 Architecture Updates", section 6.1 (cumulative decay) and 6.6.
  // Each key channel picks the reference point of its factors:
  //  * chunk start (the common case): QG_i = s q_i Gamma_i, KG_i = k_i
  //    Gamma_i, KI_i = -k_i / Gamma_i.  Safe while Gamma_L >= 2^-100, which
  //    holds when every 16-token block decays by at most 2^-25;
  //  * block start, when some block of the channel decays more:
  //    Pi_i = Gamma_i / Gamma_{16b-1} (b the token's 16-token block) in place
  //    of Gamma_i.  Pi stays within [T_b, 1] (T_b the block's decay), so the
  //    operands stay in range however much the chunk decays as a whole; the
  //    rest of each ratio is a product over whole blocks, which the tiles
  //    (F_IJ) and the state products (P_b) apply per channel.
  // KIT = -K_end^T, K_end_i = k_i Gamma_L / Gamma_i, in either form.  Returns
  // (wave-uniform) bit 0: some block decays below 2^KDA_BLOCK_LOG2_MIN, past
  // what the block-start reference can scale; bits 1-2: the wave's reference
  // mode (KDA_MODE_*).
  static __device__ __forceinline__ int prep(const Raw& r, LDS char* smem, float scale,
                                             const Prologue& pro, float ea, int hi,
                                             const PrepAddr& pa) {
    if constexpr (Cfg::SG) {
      prep_sg(r, smem, scale, pro, ea, hi);
      return 0;
    } else {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const int tg = l / CQ, cq = l % CQ;
    const int kc0 = w * (DK / NW) + CPL * cq;
    const int vc0 = w * VW + VPL * cq;
    constexpr int GPB = 16 / TPL;               // token groups per 16-token block
    static_assert(CQ == TPL && CQ * GPB == 16, "a 16-token block is one 16-lane row");
    const int blk = tg / GPB;
    LDS T* QG = (LDS T*)(smem + Cfg::OFF_QG);
    LDS T* KG = (LDS T*)(smem + Cfg::OFF_KG);
    LDS T* KI = (LDS T*)(smem + Cfg::OFF_KI);
    LDS T* BV = (LDS T*)(smem + Cfg::OFF_BV);
    LDS T* KIT = (LDS T*)(smem + Cfg::OFF_KT);
    LDS float* GL = (LDS float*)(smem + Cfg::OFF_GL);
    LDS float* BT = (LDS float*)(smem + Cfg::OFF_BT);
    LDS float* DT = (LDS float*)(smem + Cfg::OFF_DT);
    LDS float* FA = (LDS float*)(smem + Cfg::OFF_FA);
    LDS float* FM = (LDS float*)(smem + Cfg::OFF_FM);
    LDS float* DP = (LDS float*)(smem + Cfg::OFF_DP);
    LDS float* DF = (LDS float*)(smem + Cfg::OFF_DF);
    LDS uint16_t* MK = (LDS uint16_t*)(smem + Cfg::OFF_MK);

    // beta is applied to R and Y later, where it scales whole rows (R =
    // Diag(beta) strict_tril(...), Ebar = Diag(beta)(v - (k Gamma) S))
    if (w == 0) {                               // lane l holds beta of token l
      BT[l] = (Cfg::FU && (pro.flags & PRO_BETA_SIGMOID)) ? sigmoid_f(r.beta) : r.beta;
    }
    // gate transform (FU): the raw gate through -5 sigmoid(exp(A_log) (g + bias)).
    // Rows past hi read as zeros and must stay identity tokens (alpha = 1),
    // so the transform leaves their gate at 0.
    const bool xg = Cfg::FU && (pro.flags & PRO_GATE);
    float gbias[CPL];
    if (xg) {
      const LDS float* GB = (const LDS float*)(smem + Cfg::OFF_NM + 2 * C * NW * 4);
      const f32x4 b0 = *lds_ptr<const f32x4>(GB + kc0), b1 = *lds_ptr<const f32x4>(GB + kc0 + 4);
      gbias[0] = b0[0]; gbias[1] = b0[1]; gbias[2] = b0[2]; gbias[3] = b0[3];
      gbias[4] = b1[0]; gbias[5] = b1[1]; gbias[6] = b1[2]; gbias[7] = b1[3];
    }

    // log2 Pi of the lane's tokens: running sums of log2 alpha over its TPL
    // tokens, then a sum scan over the block's token groups (one DPP row) and
    // one group back; the block's last group holds log2 T_b.
    constexpr float LOG2E = 1.4426950408889634f;
    float ls[TPL][CPL];
#pragma unroll
    for (int t = 0; t < TPL; ++t)
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float gr = __uint_as_float(r.g[t].word(c));
        const bool real = TPL * tg + t < hi;
        const float la = (xg ? (real ? gate_logalpha(gr, ea, gbias[c]) : 0.f) : gr) * LOG2E;
        ls[t][c] = (t == 0) ? la : ls[t - 1][c] + la;
      }
    float ex[CPL], tb[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      tb[c] = row_scan<CQ>(ls[TPL - 1][c]);
      ex[c] = dpp_row_shr0<CQ>(tb[c]);
    }
    if (tg % GPB == GPB - 1) {
      LDS float* dt = (LDS float*)(smem + Cfg::OFF_DT + pa.fac);
      *lds_ptr<f32x4>(dt) = f32x4{tb[0], tb[1], tb[2], tb[3]};
      *lds_ptr<f32x4>(dt + 8) = f32x4{tb[4], tb[5], tb[6], tb[7]};
    }
    // -v and the unpacked q (work without decay factors, while the block
    // totals reach LDS)
    float qv[TPL][CPL];
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      st_neg((LDS T*)(smem + Cfg::OFF_BV + pa.rowv) + t * Cfg::LD_V, r.v[t]);   // -v: sign bits flipped
      r.q[t].unpack(qv[t]);
    }
    __asm__ __volatile__("" ::: "memory");

    // The block factors, one (block, channel) pair of the wave per lane (a
    // wave's LDS accesses complete in order; each wave reads back only its
    // own channels), from the log2 block totals l_0 .. l_3 of the channel.
    // A channel takes block-start references if one of its blocks decays by
    // more than 2^KDA_CHUNK_REF_LOG2_MIN (chunk-start references then stay
    // above Gamma_L >= 2^-100):
    //   chunk start: FA = P_b, FM = Gamma_L;  block start: FA = 1, FM = TQ_b
    // with TQ_b = T_b .. T_3, and for the other waves Gamma_L, P_b and F_bJ
    // (1 for chunk-referenced channels) and the channel mask.  A chunk with a
    // block below 2^KDA_BLOCK_LOG2_MIN is flagged for the token-by-token path.
    constexpr int CW = DK / NW, NPASS = (4 * CW + 63) / 64;
    float lt[NPASS][4];
    bool bref[NPASS];
    bool any_ref = false, any_scale = false, gone = false;
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int pp = 64 * ps + l;
      const int pc = frag_pos(w * CW + (pp % CW));
#pragma unroll
      for (int b = 0; b < 4; ++b) lt[ps][b] = (pp < 4 * CW) ? DT[b * DK + pc] : 0.f;
      const float mn = fminf(fminf(lt[ps][0], lt[ps][1]), fminf(lt[ps][2], lt[ps][3]));
      bref[ps] = !(mn >= KDA_CHUNK_REF_LOG2_MIN);
      any_ref |= bref[ps];
      any_scale |= bref[ps] && !(lt[ps][0] < KDA_STATE_LOG2_NEGLIGIBLE);
      gone |= !(mn >= KDA_BLOCK_LOG2_MIN);
    }
    const int mode = __any(any_scale) ? KDA_MODE_SCALE : __any(any_ref) ? KDA_MODE_MASK
                                                                         : KDA_MODE_CHUNK;
    const bool bad = __any(gone);
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
      const int pp = 64 * ps + l;
      if (pp < 4 * CW) {
        const int b = pp / CW, c = w * CW + pp % CW, pc = frag_pos(c);
        const float l0 = lt[ps][0], l1 = lt[ps][1], l2 = lt[ps][2], l3 = lt[ps][3];
        const bool c1 = b >= 1, c2 = b >= 2, c3 = b == 3;
        const float lp = (c1 ? l0 : 0.f) + (c2 ? l1 : 0.f) + (c3 ? l2 : 0.f);
        const float lg = (l0 + l1) + (l2 + l3);
        const float gf = __builtin_amdgcn_exp2f(lg);
        if (!bref[ps]) {
          FA[b * DK + pc] = __builtin_amdgcn_exp2f(lp);
          FM[b * DK + pc] = gf;
          if (c1) {
            DP[b * DK + pc] = 1.f;
            const int pb0 = b * (b - 1) / 2;
            DF[(pb0 + b - 1) * DK + pc] = 1.f;
            if (c2) DF[(pb0 + b - 2) * DK + pc] = 1.f;
            if (c3) DF[pb0 * DK + pc] = 1.f;
          }
        } else {
          FA[b * DK + pc] = 1.f;
          FM[b * DK + pc] = __builtin_amdgcn_exp2f(lg - lp);
          if (c1) {
            DP[b * DK + pc] = __builtin_amdgcn_exp2f(lp);
            // F_{b,b-1} = T_{b-1}, F_{b,b-2} = T_{b-2} T_{b-1}, F_{3,0} = T_0 T_1 T_2
            const float lm1 = c3 ? l2 : (c2 ? l1 : l0);
            const float lm2 = c3 ? l1 : l0;
            const int pb0 = b * (b - 1) / 2;
            DF[(pb0 + b - 1) * DK + pc] = __builtin_amdgcn_exp2f(lm1);
            if (c2) DF[(pb0 + b - 2) * DK + pc] = __builtin_amdgcn_exp2f(lm2 + lm1);
            if (c3) DF[pb0 * DK + pc] = __builtin_amdgcn_exp2f(lp);
          }
        }
        if (b == 0) {
          GL[c] = gf;
          MK[pc] = bref[ps] ? (uint16_t)0 : (uint16_t)0xffff;
        }
      }
    }
    __asm__ __volatile__("" ::: "memory");
    // the lane's factors (issued now, used after the k work below)
    const LDS float* fap = (const LDS float*)(smem + Cfg::OFF_FA + pa.fac);
    const LDS float* fmp = (const LDS float*)(smem + Cfg::OFF_FM + pa.fac);
    const f32x4 fa0 = *lds_ptr<const f32x4>(fap), fa1 = *lds_ptr<const f32x4>(fap + 8);
    const f32x4 fm0 = *lds_ptr<const f32x4>(fmp), fm1 = *lds_ptr<const f32x4>(fmp + 8);
    __asm__ __volatile__("" ::: "memory");
    // k unpacked, and the L2 norms (FU)
    float kv[TPL][CPL];
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      const int i = TPL * tg + t;
      r.k[t].unpack(kv[t]);
      if (Cfg::FU && (pro.flags & PRO_L2NORM)) {
        // the token's squared norms: the sum of the waves' partials
        const LDS float* NQ = (const LDS float*)(smem + Cfg::OFF_NM) + i * NW;
        const LDS float* NK = NQ + C * NW;
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int j = 0; j < NW; j += 4) {
          const f32x4 a = *lds_ptr<const f32x4>(NQ + j), b = *lds_ptr<const f32x4>(NK + j);
          sq += (a[0] + a[1]) + (a[2] + a[3]);
          sk += (b[0] + b[1]) + (b[2] + b[3]);
        }
        const float rq = __builtin_amdgcn_rsqf(sq + PRO_NORM_EPS);
        const float rk = __builtin_amdgcn_rsqf(sk + PRO_NORM_EPS);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          qv[t][c] *= rq;
          kv[t][c] *= rk;
        }
      }
    }
    const float fa[CPL] = {fa0[0], fa0[1], fa0[2], fa0[3], fa1[0], fa1[1], fa1[2], fa1[3]};
    const float fm[CPL] = {fm0[0], fm0[1], fm0[2], fm0[3], fm1[0], fm1[1], fm1[2], fm1[3]};

    // the operands; -K_end of the lane's tokens per key channel for the
    // key-major copy
    constexpr bool KIT_PAIRS = Cfg::SZ == 2 && TPL == 2;
    T kit[CPL][TPL];
    float kef[CPL][TPL];
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
      const int i = TPL * tg + t;
      float qg[CPL], kg[CPL], ki[CPL];
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const float gam = __builtin_amdgcn_exp2f(ex[c] + ls[t][c]) * fa[c];
        const float inv = __builtin_amdgcn_rcpf(gam);
        qg[c] = scale * qv[t][c] * gam;
        kg[c] = kv[t][c] * gam;                 // beta comes later
        ki[c] = -kv[t][c] * inv;
        kef[c][t] = ki[c] * fm[c];              // -K_end
        kit[c][t] = Op::cvt(kef[c][t]);
      }
      st8_at((LDS T*)(smem + Cfg::OFF_QG + pa.rowk) + t * Cfg::LD_K, qg);
      st8_at((LDS T*)(smem + Cfg::OFF_KG + pa.rowk) + t * Cfg::LD_K, kg);
      st8_at((LDS T*)(smem + Cfg::OFF_KI + pa.rowk) + t * Cfg::LD_K, ki);
    }
    // key-major copy KIT[channel][token]: the lane's TPL tokens are
    // consecutive (and stay so under the token permutation)
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      LDS T* p = (LDS T*)(smem + Cfg::OFF_KT + pa.kit) + c * Cfg::LD_KT;
      if (KIT_PAIRS)
        *lds_ptr<uint32_t>(p) = pack_bf16x2(kef[c][0], kef[c][TPL - 1]);
      else
        st_vec(p, kit[c]);
    }
    return (bad ? 1 : 0) | (mode << 1);
    }
  }

  // N raw input elements to LDS with their sign bits flipped (exact negation;
  // the I/O type equals the operand type wherever this is used)
  template <int N>
  static __device__ __forceinline__ void st_neg(LDS T* p, const RawIo<Io, N>& x) {
    static_assert(sizeof(typename Io::storage) == sizeof(T), "raw words are operand words");
    constexpr int W = N * (int)sizeof(T) / 4;
    constexpr uint32_t SIGN = sizeof(T) == 2 ? 0x80008000u : 0x80000000u;
#pragma unroll
    for (int i = 0; i < W; i += 4) {
      if (W - i >= 4) {
        *lds_ptr<u32x4>(p + i * 4 / (int)sizeof(T)) =
            u32x4{x.w.word(i) ^ SIGN, x.w.word(i + 1) ^ SIGN, x.w.word(i + 2) ^ SIGN, x.w.word(i + 3) ^ SIGN};
      } else if (W - i == 2) {
        *lds_ptr<u32x2>(p + i * 4 / (int)sizeof(T)) = u32x2{x.w.word(i) ^ SIGN, x.w.word(i + 1) ^ SIGN};
      } else {
        *lds_ptr<uint32_t>(p + i * 4 / (int)sizeof(T)) = x.w.word(i) ^ SIGN;
      }
    }
  }

  // Channels c0 .. c0+7 of one row from floats: bf16 pairs packed straight
  // into words (round to nearest even, as Op::cvt) and stored at their
  // permuted positions; fp32 as they are.
  static __device__ __forceinline__ void st_row8(LDS T* row, int c0, const float (&x)[8]) {
    if (Op::PERMUTED) {
      *lds_ptr<u32x2>(row + Op::perm_pos(c0)) = u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
      *lds_ptr<u32x2>(row + Op::perm_pos(c0 + 4)) =
          u32x2{pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])};
    } else {
      T y[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) y[c] = Op::cvt(x[c]);
      st_chunk(row + c0, y);
    }
  }

  // 8 consecutive channels c0 .. c0+7 of one row of a channel-permuted
  // buffer: two 4-element pieces at their permuted positions
  static __device__ __forceinline__ void st_perm(LDS T* row, int c0, const T (&x)[8]) {
    if (!Op::PERMUTED) { st_chunk(row + c0, x); return; }
    const T a[4] = {x[0], x[1], x[2], x[3]}, b[4] = {x[4], x[5], x[6], x[7]};
    st_vec(row + Op::perm_pos(c0), a);
    st_vec(row + Op::perm_pos(c0 + 4), b);
  }

  // N elements to LDS as 16-byte (or smaller) vector stores
  template <int N>
  static __device__ __forceinline__ void st_chunk(LDS T* p, const T (&x)[N]) {
    constexpr int PER = 16 / (int)sizeof(T) < N ? 16 / (int)sizeof(T) : N;
#pragma unroll
    for (int c0 = 0; c0 < N; c0 += PER) {
      T part[PER];
#pragma unroll
      for (int c = 0; c < PER; ++c) part[c] = x[c0 + c];
      st_vec(p + c0, part);
    }
  }

  // A 32-deep operand fragment over key channels 32 ks .. 32 ks + 31 with the
  // lane's block-referenced channels zeroed (the channel mask holds 16-bit
  // all-ones or zeros in fragment order, one 16-byte read per lane).
  static __device__ __forceinline__ typename Op::F32 mask_frag(LDS char* smem, typename Op::F32 f,
                                                                int ks, int l) {
    const LDS uint16_t* MK = (const LDS uint16_t*)(smem + Cfg::OFF_MK) + 32 * ks + 8 * (l >> 4);
    if constexpr (Cfg::SZ == 2) {
      const u32x4 m = *lds_ptr<const u32x4>(MK);
      const u32x2 a = __builtin_bit_cast(u32x2, f.lo), b = __builtin_bit_cast(u32x2, f.hi);
      f.lo = __builtin_bit_cast(typename Op::F16, u32x2{a[0] & m[0], a[1] & m[1]});
      f.hi = __builtin_bit_cast(typename Op::F16, u32x2{b[0] & m[2], b[1] & m[3]});
    } else {
      const u32x4 m = *lds_ptr<const u32x4>(MK);
      f32x4 lo = f.lo, hi = f.hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = ((m[e >> 1] >> (16 * (e & 1))) & 0xffffu) ? lo[e] : 0.f;
        hi[e] = ((m[2 + (e >> 1)] >> (16 * (e & 1))) & 0xffffu) ? hi[e] : 0.f;
      }
      f.lo = lo;
      f.hi = hi;
    }
    return f;
  }

  // ---------------------------------------------------------------- phase A
  // R = strict_tril(KG KI^T) and Aqk = tril(QG KI^T) by 16x16 tiles, from
  // the stored -KI (so the products come out negated).  KDA: the operands
  // are referenced to their own block's start, so a tile across blocks (I >
  // J) takes the decay of the whole blocks J .. I-1 between the two
  // references (F_IJ, per key channel) on its -KI fragments.  The tiles are formed
  // as (KI QG^T)^T-style products so that a lane ends up with four
  // consecutive columns of one row: off-diagonal -R tiles go row-major to RR,
  // -Aqk row-major to AQ (columns permuted like the 32-deep operand that reads
  // them), and the diagonal R tiles (in the other orientation) to RD, fp32,
  // column-contiguous, for the inverse.
  // MODE (KDA_MODE_*): whether some channel is block-referenced, so that the
  // cross-block tiles take F_IJ.
  template <int MODE>
  static __device__ __forceinline__ void tile_qk(LDS char* smem, int I, int J) {
    const int l = lane_fresh();
    const LDS T* QG = (const LDS T*)(smem + Cfg::OFF_QG);
    const LDS T* KG = (const LDS T*)(smem + Cfg::OFF_KG);
    const LDS T* KI = (const LDS T*)(smem + Cfg::OFF_KI);
    LDS T* RR = (LDS T*)(smem + Cfg::OFF_RT);
    LDS T* AQ = (LDS T*)(smem + Cfg::OFF_AQ);
    LDS float* RD = (LDS float*)(smem + Cfg::OFF_RD);
    f32x4 accR = {0.f, 0.f, 0.f, 0.f}, accA = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      typename Op::F32 b = Op::ld32_rmp(l, KI, Cfg::LD_K, 16 * J, 32 * ks);
      if constexpr (!Cfg::SG) {
        if (MODE != KDA_MODE_CHUNK && I != J) {
          const LDS float* F = (const LDS float*)(smem + Cfg::OFF_DF) +
                               (I * (I - 1) / 2 + J) * DK + 32 * ks + 8 * (l >> 4);
          b.lo = Op::pack(Op::unpack(b.lo) * *lds_ptr<const f32x4>(F));
          b.hi = Op::pack(Op::unpack(b.hi) * *lds_ptr<const f32x4>(F + 4));
        }
      }
      const typename Op::F32 ak = Op::ld32_rmp(l, KG, Cfg::LD_K, 16 * I, 32 * ks);
      const typename Op::F32 aq = Op::ld32_rmp(l, QG, Cfg::LD_K, 16 * I, 32 * ks);
      accR = (I == J) ? Op::mma32(ak, b, accR) : Op::mma32(b, ak, accR);
      accA = Op::mma32(b, aq, accA);
    }
    // accA[r] = -Aqk[16I + n][16J + g4 + r]; accR[r] = -R[16I + g4 + r][16I + n]
    // on the diagonal, -R[16I + n][16J + g4 + r] off it, once the rows are
    // scaled by beta
    const int n = l & 15, g4 = 4 * (l >> 4);
    const LDS float* BT = (const LDS float*)(smem + Cfg::OFF_BT);
    if constexpr (Cfg::SG) {
      // raw products: entry (i, j) of -R takes beta_i rk_i rk_j Gamma_i/Gamma_j,
      // of -Aqk rq_i rk_j Gamma_i/Gamma_j; masked entries are selected away
      // before the (possibly overflowing) ratio is used
      const LDS float* SV = (const LDS float*)(smem + Cfg::OFF_SV);
      if (I == J) {
        // accR[r]: i = 16I + g4 + r, j = 16I + n; accA[r]: i = 16I + n, j = 16I + g4 + r
        const f32x4 gr = *lds_ptr<const f32x4>(SV + SV_G * C + 16 * I + g4);
        const f32x4 br = *lds_ptr<const f32x4>(SV + SV_BK * C + 16 * I + g4);
        const f32x4 kr = *lds_ptr<const f32x4>(SV + SV_RK * C + 16 * I + g4);
        const float gn = SV[SV_G * C + 16 * I + n], kn = SV[SV_RK * C + 16 * I + n];
        const float qn = SV[SV_RQ * C + 16 * I + n];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float fr = __builtin_amdgcn_exp2f(gr[r] - gn) * br[r] * kn;
          const float fa = __builtin_amdgcn_exp2f(gn - gr[r]) * qn * kr[r];
          accR[r] = (n < g4 + r) ? accR[r] * fr : 0.f;    // strictly lower
          accA[r] = (g4 + r <= n) ? accA[r] * fa : 0.f;   // lower with diagonal
        }
      } else {
        // i = 16I + n, j = 16J + g4 + r for both; gamma_i - gamma_j = gi +
        // (rest of block J after j) + (whole blocks between), all block-local
        const f32x4 gj = *lds_ptr<const f32x4>(SV + SV_G * C + 16 * J + g4);
        const f32x4 kj = *lds_ptr<const f32x4>(SV + SV_RK * C + 16 * J + g4);
        const float gi = SV[SV_G * C + 16 * I + n], bi = SV[SV_BK * C + 16 * I + n];
        const float qi = SV[SV_RQ * C + 16 * I + n];
        const float tj = SV[SV_T * C + J];
        float mid = 0.f;
        for (int b = J + 1; b < I; ++b) mid += SV[SV_T * C + b];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(gi + ((tj - gj[r]) + mid)) * kj[r];
          accR[r] *= e * bi;
          accA[r] *= e * qi;
        }
      }
    } else {
      if (I == J)
        accR *= *lds_ptr<const f32x4>(BT + 16 * I + g4);
      else
        accR *= BT[16 * I + n];
      if (I == J) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (!(n < g4 + r)) accR[r] = 0.f;    // strictly lower
          if (!(g4 + r <= n)) accA[r] = 0.f;   // lower with diagonal
        }
      }
    }
    if (I == J) {
      // RD[I][m][i] = R[16I + i][16I + m]  (column m of the block, contiguous over i)
      *lds_ptr<f32x4>(RD + I * 16 * Cfg::RD_LD + n * Cfg::RD_LD + g4) = -accR;
    } else {
      *lds_ptr<typename Op::F16>(RR + (16 * I + n) * Cfg::LD_RR + 16 * J + g4) = Op::pack(accR);
    }
    *lds_ptr<typename Op::F16>(AQ + (16 * I + n) * Cfg::LD_AQ + Op::perm_pos(16 * J + g4)) =
        Op::pack(accA);
  }

  // ---------------------------------------------------------------- phase T
  // T_II = (I + R_II)^{-1} for diagonal block BLK, by column forward
  // substitution: lane col (< 16) holds column col.  Written transposed
  // (TD[BLK][col][i]).
  template <int BLK>
  static __device__ __forceinline__ void invert_diag(LDS char* smem) {
    const int l = lane_fresh();
    const int col = l & 15, blk = BLK;
    const LDS float* RD = (const LDS float*)(smem + Cfg::OFF_RD) + blk * 16 * Cfg::RD_LD;
    LDS T* TD = (LDS T*)(smem + Cfg::OFF_TD) + blk * 256;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (i == col) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < 15; ++m) {
      const float xm = x[m];
      // column m of N: N[i][m] = RD[m][i]
#pragma unroll
      for (int i4 = (m + 1) / 4; i4 < 4; ++i4) {
        const f32x4 nv = *lds_ptr<const f32x4>(RD + m * Cfg::RD_LD + 4 * i4);
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

  // ---------------------------------------------------------------- phase S
  // Y = -Ebar = Diag(beta) (KG S - V); X = (I + R)^{-1} Y = -E by block
  // forward substitution; O^T = S^T QG^T + (-E)^T (-Aqk)^T staged through LDS
  // and written as whole token rows; S <- Diag(Gamma_L) (S + (-KI)^T (-E)).
  // The parts that need no inverse: Y_I = Diag(beta_I) (KG_I S - V_I) and the S part of
  // the outputs, O_I^T = S^T QG_I^T, for the four token blocks, with S as
  // 32-deep operands over key channels (lane: value column, k: channels).
  // KDA: block-referenced channels take the state into block I's products as
  // Diag(P_I) S (P_I = T_0 .. T_{I-1}; 1 for the others), or drop out of
  // blocks 1 .. 3 when P_1 is negligible (MODE).
  template <int MODE>
  static __device__ __forceinline__ void scan_y(LDS char* smem, const f32x4 (&S)[MTK][NVT],
                                                f32x4 (&Y)[4][NVT], f32x4 (&O)[4][NVT]) {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const LDS T* KG = (const LDS T*)(smem + Cfg::OFF_KG);
    const LDS T* QG = (const LDS T*)(smem + Cfg::OFF_QG);
    const LDS T* BV = (const LDS T*)(smem + Cfg::OFF_BV);
    const LDS float* BT = (const LDS float*)(smem + Cfg::OFF_BT);
    const LDS float* DP = (const LDS float*)(smem + Cfg::OFF_DP);
    typename Op::F32 SB[NKS][NVT];
    const int vw0 = w * VW;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      if (I == 0 || (!Cfg::SG && MODE == KDA_MODE_SCALE)) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) {
            f32x4 lo = S[2 * ks][nt], hi = S[2 * ks + 1][nt];
            if (!Cfg::SG && MODE == KDA_MODE_SCALE && I > 0) {
              // rows 32 ks + 4g + r and 32 ks + 16 + 4g + r: fragment positions
              // 32 ks + 8g + r and 32 ks + 8g + 4 + r
              const LDS float* P = DP + I * DK + 32 * ks + 8 * (l >> 4);
              lo *= *lds_ptr<const f32x4>(P);
              hi *= *lds_ptr<const f32x4>(P + 4);
            }
            SB[ks][nt] = typename Op::F32{Op::pack(lo), Op::pack(hi)};
          }
      } else if (!Cfg::SG && MODE == KDA_MODE_MASK && I == 1) {
        // blocks 1 .. 3: the block-referenced rows of S drop out (P_I < 2^-40)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) SB[ks][nt] = mask_frag(smem, SB[ks][nt], ks, l);
      }
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt)
        Y[I][nt] = Op::unpack(Op::ld16_tr(l, BV, Cfg::LD_V, 16 * I, vw0 + 16 * nt));   // -V
      const f32x4 b = *lds_ptr<const f32x4>(BT + 16 * I + 4 * (l >> 4));
      if constexpr (Cfg::SG) {
        // raw k: Y = Diag(beta) (-v) + Diag(beta Gamma rk) (k S)
        const LDS float* SV = (const LDS float*)(smem + Cfg::OFF_SV);
        const f32x4 fy = *lds_ptr<const f32x4>(SV + SV_FY * C + 16 * I + 4 * (l >> 4));
        f32x4 Z[NVT];
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) Z[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const typename Op::F32 ak = Op::ld32_rmp(l, KG, Cfg::LD_K, 16 * I, 32 * ks);
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) Z[nt] = Op::mma32(ak, SB[ks][nt], Z[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) Y[I][nt] = Y[I][nt] * b + Z[nt] * fy;
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const typename Op::F32 ak = Op::ld32_rmp(l, KG, Cfg::LD_K, 16 * I, 32 * ks);
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) Y[I][nt] = Op::mma32(ak, SB[ks][nt], Y[I][nt]);
        }
        // rows 16I + g4 + r scaled by beta: Y = Diag(beta)((k Pi) (P_I S) - v)
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) Y[I][nt] *= b;
      }
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) O[I][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const typename Op::F32 bq = Op::ld32_rmp(l, QG, Cfg::LD_K, 16 * I, 32 * ks);
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) O[I][nt] = Op::mma32(SB[ks][nt], bq, O[I][nt]);
      }
      if constexpr (Cfg::SG) {
        // column n = token 16I + n: raw q, so S^T q_i takes Gamma_i rq_i
        const float fo = ((const LDS float*)(smem + Cfg::OFF_SV))[SV_FO * C + 16 * I + (l & 15)];
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) O[I][nt] *= fo;
      }
    }
  }

  // next_norms: also write the next chunk's norm partials from `nxt` (FU with
  // the L2-norm transform), ahead of the barrier this step has anyway.
  static __device__ __forceinline__ void scan_step(LDS char* smem, f32x4 (&S)[MTK][NVT],
                                                   f32x4 (&Y)[4][NVT], f32x4 (&Ob)[4][NVT],
                                                   void* out,
                                                   size_t row_base, int H, int h, int clen,
                                                   const Raw& nxt, bool next_norms) {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const LDS T* QG = (const LDS T*)(smem + Cfg::OFF_QG);
    const LDS T* KG = (const LDS T*)(smem + Cfg::OFF_KG);
    const LDS T* KIT = (const LDS T*)(smem + Cfg::OFF_KT);
    const LDS T* BV = (const LDS T*)(smem + Cfg::OFF_BV);
    const LDS T* AQ = (const LDS T*)(smem + Cfg::OFF_AQ);
    const LDS T* RR = (const LDS T*)(smem + Cfg::OFF_RT);
    const LDS T* TD = (const LDS T*)(smem + Cfg::OFF_TD);
    LDS T* OST = (LDS T*)(smem + Cfg::OFF_OS);
    const LDS float* GL = (const LDS float*)(smem + Cfg::OFF_GL);
    const int vw0 = w * VW;
    const int g4 = 4 * (l >> 4);

    // (2) the solve X_I = T_II (Y_I - sum_{J<I} R_IJ X_J) by 16-token
    //     blocks; X kept as 16-deep operands.
    typename Op::F16 XP[4][NVT];
    // SG: X rows scaled by rk_j Gamma_L / Gamma_j for the update of S from the raw k
    typename Op::F16 XS[Cfg::SG ? 4 : 1][NVT];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 (&YI)[NVT] = Y[I];
      // The -R_IJ X_J terms accumulate in their own registers (16-deep
      // products) and join Y with a vector add: an accumulator produced by
      // one MFMA shape is never fed straight into another shape's
      // accumulate input.  Mixed-shape accumulation chains were miscompiled
      // for gfx950 (too few wait states after the 32-deep producer).
      if (I > 0) {
        f32x4 Z[NVT];
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) Z[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < I; ++J) {
          // A[m = i][k = j] = -R[16I + m][16J + k] = RR[16I + m][16J + k]
          const typename Op::F16 a = Op::ld16_rm(l, RR, Cfg::LD_RR, 16 * I, 16 * J);
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) Z[nt] = Op::mma16(a, XP[J][nt], Z[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) YI[nt] += Z[nt];
      }
      // A[m = i][k = i'] = T_II[m][k] = TD[I][k][m]
      const typename Op::F16 a = Op::ld16_tr(l, TD + I * 256, 16, 0, 0);
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 x = Op::mma16(a, Op::pack(YI[nt]), z);
        XP[I][nt] = Op::pack(x);
        if constexpr (Cfg::SG) {
          const f32x4 fs = *lds_ptr<const f32x4>((const LDS float*)(smem + Cfg::OFF_SV) +
                                                 SV_FS * C + 16 * I + g4);
          XS[I][nt] = Op::pack(x * fs);
        }
      }
    }
    // -E as 32-deep operands over tokens: two 16-deep blocks side by side
    typename Op::F32 EB[2][NVT], ES[Cfg::SG ? 2 : 1][NVT];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        EB[kt][nt] = typename Op::F32{XP[2 * kt][nt], XP[2 * kt + 1][nt]};
        if constexpr (Cfg::SG)
          ES[kt][nt] = typename Op::F32{XS[2 * kt][nt], XS[2 * kt + 1][nt]};
      }

    // (3) O_I^T = S^T QG_I^T + (-E)^T (-Aqk_I)^T: rows = value columns,
    //     columns = tokens 16I + n; staged as OST[token][value]
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 (&O)[NVT] = Ob[I];
#pragma unroll
      for (int kt = 0; kt <= I / 2; ++kt) {
        const typename Op::F32 ba = Op::ld32_rmp(l, AQ, Cfg::LD_AQ, 16 * I, 32 * kt);
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt) O[nt] = Op::mma32(EB[kt][nt], ba, O[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) Op::st_ct(l, OST, Cfg::LD_OS, 16 * I, vw0 + 16 * nt, O[nt]);
    }
    // (4) state update, S <- Diag(Gamma_L) S + K_end^T E (section 6.4), from
    //     the key-major -K_end (KDA) or -k (Gated DeltaNet) and -E.
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt) {
      const f32x4 gl = *lds_ptr<const f32x4>(GL + 16 * mt + g4);
      typename Op::F32 a[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        a[kt] = Op::ld32_rmp(l, KIT, Cfg::LD_KT, 16 * mt, 32 * kt);
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        if constexpr (Cfg::SG) {
          // S <- Gamma_L S + (-k)^T (-E rk Gamma_L / Gamma)
          f32x4 s = S[mt][nt] * gl;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) s = Op::mma32(a[kt], ES[kt][nt], s);
          S[mt][nt] = s;
        } else {
          f32x4 s = S[mt][nt] * gl;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) s = Op::mma32(a[kt], EB[kt][nt], s);
          S[mt][nt] = s;
        }
      }
    }
    // The next chunk's q and k have arrived by now (loaded before the last
    // barrier); their norm partials go to LDS here, where no wave reads them
    // any more, and are visible to the next prep after the barrier below.
    if (Cfg::FU && next_norms) norm_partials(nxt, smem);
    // Once the staged tile is complete all of the chunk's LDS reads are done:
    // after this barrier only the copy below reads LDS, and the next chunk's
    // prep writes nothing it reads, so no barrier separates the two.
    __syncthreads();
    // copy the staged tile out: 16-byte pieces of whole token rows
    {
      constexpr int PIECE = 16 / Cfg::SZ;                 // elements per 16 bytes
      constexpr int PER_ROW = DV / PIECE;
      constexpr uint32_t E = sizeof(typename Io::storage);
      const uint32_t srow = (uint32_t)H * DV * E;
      const __amdgpu_buffer_rsrc_t ro =
          make_rsrc((char*)out + (row_base * H + h) * DV * E, clen * srow);
#pragma unroll
      for (int p0 = 0; p0 < C * PER_ROW; p0 += Cfg::NTHREADS) {
        const int p = p0 + threadIdx.x;
        const int i = p / PER_ROW, c = (p % PER_ROW) * PIECE;
        const u32x4 val = *lds_ptr<const u32x4>(OST + i * Cfg::LD_OS + c);
        buf_store16(ro, i * srow + c * E, val);   // rows past clen are dropped
      }
    }

  }

  // ---------------------------------------------------------------- guard path
  // The recurrence itself, token by token, on the on-chip state (each wave its
  // own value columns; reductions over key rows stay inside the wave).
  static __device__ __forceinline__ void recurrent_chunk(f32x4 (&S)[MTK][NVT], const void* q,
                                                         const void* k, const void* v,
                                                         const float* g, const float* beta,
                                                         void* out, size_t row_base, int H,
                                                         int h, int clen, float scale,
                                                         const Prologue& pro, float ea,
                                                         int vw0 = -1) {
    // vw0: the first value column of this wave's state tiles (default: the
    // wave's own slice of the workgroup)
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const int n = l & 15, g4 = 4 * (l >> 4);
    if (vw0 < 0) vw0 = w * VW;
    const bool xg = Cfg::FU && (pro.flags & PRO_GATE);
    const bool xn = Cfg::FU && (pro.flags & PRO_L2NORM);
    for (int t = 0; t < clen; ++t) {
      const size_t row = (row_base + t) * H + h;
      // forget, then the prediction Sbar^T k
      float p[NVT];
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) p[nt] = 0.f;
      float k2 = 0.f;
#pragma unroll
      for (int mt = 0; mt < MTK; ++mt) {
        const size_t ci = row * DK + 16 * mt + g4;
        f32x4 gv;
        if constexpr (Cfg::SG)
          gv = f32x4{g[row], g[row], g[row], g[row]};
        else
          gv = *reinterpret_cast<const f32x4*>(g + ci);
        const f32x4 kv = Io::load4(k, ci);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float gr = gv[r];
          if (xg) {
            const float bias =
                pro.bias ? pro.bias[Cfg::SG ? h : h * DK + 16 * mt + g4 + r] : 0.f;
            gr = gate_logalpha(gr, ea, bias);
          }
          const float a = __expf(gr);
          if (Cfg::FU) k2 += kv[r] * kv[r];
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) {
            S[mt][nt][r] *= a;
            p[nt] += S[mt][nt][r] * kv[r];
          }
        }
      }
      float b = beta[row];
      if (Cfg::FU && (pro.flags & PRO_BETA_SIGMOID)) b = sigmoid_f(b);
      // L2 norm of k (FU): the sums used the raw k; scale afterwards
      float rk = 1.f;
      if (xn) {
        k2 += __shfl_xor(k2, 16);
        k2 += __shfl_xor(k2, 32);
        rk = __builtin_amdgcn_rsqf(k2 + PRO_NORM_EPS);
      }
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        p[nt] += __shfl_xor(p[nt], 16);
        p[nt] += __shfl_xor(p[nt], 32);
        p[nt] = b * (Io::load(v, row * DV + vw0 + 16 * nt + n) - p[nt] * rk) * rk;  // e / |k|
      }
      // write k e^T, then read with s q
      float o[NVT];
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) o[nt] = 0.f;
      float q2 = 0.f;
#pragma unroll
      for (int mt = 0; mt < MTK; ++mt) {
        const size_t ci = row * DK + 16 * mt + g4;
        const f32x4 kv = Io::load4(k, ci);
        const f32x4 qv = Io::load4(q, ci);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (Cfg::FU) q2 += qv[r] * qv[r];
#pragma unroll
          for (int nt = 0; nt < NVT; ++nt) {
            S[mt][nt][r] += kv[r] * p[nt];
            o[nt] += S[mt][nt][r] * (scale * qv[r]);
          }
        }
      }
      float rq = 1.f;
      if (xn) {
        q2 += __shfl_xor(q2, 16);
        q2 += __shfl_xor(q2, 32);
        rq = __builtin_amdgcn_rsqf(q2 + PRO_NORM_EPS);
      }
#pragma unroll
      for (int nt = 0; nt < NVT; ++nt) {
        o[nt] += __shfl_xor(o[nt], 16);
        o[nt] += __shfl_xor(o[nt], 32);
        if (l < 16) Io::store(out, row * DV + vw0 + 16 * nt + n, o[nt] * rq);
      }
    }
  }

  // ---------------------------------------------------------------- middle interval
  // One interval for the tiles, the inverses and the products that need no
  // inverse: wave I < 4 forms diagonal tile (I, I) and inverts it itself (one
  // wave's LDS accesses complete in order), waves 4-7 form the six
  // off-diagonal pairs; each wave's case is one scheduling region, so VALU
  // (inverse) and MFMA (tiles, Y, S^T QG^T) interleave.
  template <int MODE>
  static __device__ __forceinline__ void middle(LDS char* smem, f32x4 (&S)[MTK][NVT],
                                                f32x4 (&Y)[4][NVT], f32x4 (&O)[4][NVT]) {
    const int w = threadIdx.x >> 6;
    if (NW == 8) {
      switch (__builtin_amdgcn_readfirstlane(w)) {
        case 0: tile_qk<MODE>(smem, 0, 0); invert_diag<0>(smem); scan_y<MODE>(smem, S, Y, O); break;
        case 1: tile_qk<MODE>(smem, 1, 1); invert_diag<1>(smem); scan_y<MODE>(smem, S, Y, O); break;
        case 2: tile_qk<MODE>(smem, 2, 2); invert_diag<2>(smem); scan_y<MODE>(smem, S, Y, O); break;
        case 3: tile_qk<MODE>(smem, 3, 3); invert_diag<3>(smem); scan_y<MODE>(smem, S, Y, O); break;
        case 4: tile_qk<MODE>(smem, 1, 0); tile_qk<MODE>(smem, 3, 2); scan_y<MODE>(smem, S, Y, O); break;
        case 5: tile_qk<MODE>(smem, 2, 0); tile_qk<MODE>(smem, 2, 1); scan_y<MODE>(smem, S, Y, O); break;
        case 6: tile_qk<MODE>(smem, 3, 0); scan_y<MODE>(smem, S, Y, O); break;
        default: tile_qk<MODE>(smem, 3, 1); scan_y<MODE>(smem, S, Y, O); break;
      }
    } else {
      switch (__builtin_amdgcn_readfirstlane(w)) {
        case 0: tile_qk<MODE>(smem, 0, 0); invert_diag<0>(smem); tile_qk<MODE>(smem, 1, 0);
                tile_qk<MODE>(smem, 2, 0); scan_y<MODE>(smem, S, Y, O); break;
        case 1: tile_qk<MODE>(smem, 1, 1); invert_diag<1>(smem); tile_qk<MODE>(smem, 2, 1);
                tile_qk<MODE>(smem, 3, 0); scan_y<MODE>(smem, S, Y, O); break;
        case 2: tile_qk<MODE>(smem, 2, 2); invert_diag<2>(smem); tile_qk<MODE>(smem, 3, 1);
                scan_y<MODE>(smem, S, Y, O); break;
        default: tile_qk<MODE>(smem, 3, 3); invert_diag<3>(smem); tile_qk<MODE>(smem, 3, 2);
                 scan_y<MODE>(smem, S, Y, O); break;
      }
    }
  }

  // ---------------------------------------------------------------- driver
  static __device__ __forceinline__ void run(const void* q, const void* k, const void* v,
                                             const float* g, const float* beta, const float* S0,
                                             void* out, float* S_final, size_t row_base, int len,
                                             int H, int h, size_t chain, float scale,
                                             const Prologue& pro) {
    extern __shared__ __attribute__((aligned(16))) char smem_[];
    LDS char* smem = (LDS char*)smem_;
    const int w = threadIdx.x >> 6;
    const int vw0 = w * VW;
    LDS int* FL = (LDS int*)(smem + Cfg::OFF_FL);

    // -Aqk tiles above the diagonal are read (inside 32-deep operands) but never
    // written: zero the buffer once.
    {
      LDS T* AQ = (LDS T*)(smem + Cfg::OFF_AQ);
      for (int i = threadIdx.x; i < C * Cfg::LD_AQ; i += Cfg::NTHREADS) AQ[i] = Op::cvt(0.f);
    }
    // FU: the head's exp(A_log) and gate biases (LDS, read by prep)
    float ea = 1.f;
    if (Cfg::FU && (pro.flags & PRO_GATE)) {
      ea = __expf(pro.A_log[h]);
      LDS float* GB = (LDS float*)(smem + Cfg::OFF_NM + 2 * C * NW * 4);
      for (int i = threadIdx.x; i < DK; i += Cfg::NTHREADS)
        GB[i] = pro.bias ? pro.bias[Cfg::SG ? h : h * DK + i] : 0.f;
      __syncthreads();
    }
    // state tiles: S[16mt + 4g + r][vw0 + 16nt + n]
    f32x4 S[MTK][NVT];
    {
      const int l = lane_fresh();
      const int n = l & 15, g4 = 4 * (l >> 4);
#pragma unroll
      for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S[mt][nt][r] = S0 ? S0[(chain * DK + 16 * mt + g4 + r) * DV + vw0 + 16 * nt + n] : 0.f;
    }

    // One register buffer of raw inputs: the prep consumes chunk c; the loads
    // of chunk c + 1 go into the same registers afterwards, spread over the
    // phases (gates after the prep, q and k after the key-key tiles, v and
    // beta after the inverse) so that the memory system sees a steady stream
    // instead of one burst per chunk that would stall the issuing waves.
    const Offsets offs = lane_offsets(H);
    const PrepAddr pa = prep_addr();
    Raw raw;
    if (len > 0) load_raw<LOAD_ALL>(raw, offs, q, k, v, g, beta, row_base, H, h, len < C ? len : C);
    const bool l2n = Cfg::FU && (pro.flags & PRO_L2NORM);
    bool norms_ready = false;   // this chunk's norm partials are in LDS already
    for (int c0 = 0; c0 < len; c0 += C) {
      const int clen = (len - c0) < C ? (len - c0) : C;
      // the next chunk's loads are issued on every step, with an empty range
      // after the last chunk (nothing is read), so that the wait before each
      // use of the raw registers only covers the loads older than it
      const bool more = c0 + C < len;
      const int nlen = !more ? 0 : ((len - c0 - C) < C ? (len - c0 - C) : C);
      const size_t next = more ? row_base + c0 + C : row_base;
      if (l2n && !norms_ready) {
        // the chunk's norms need every wave's channels: one more barrier (the
        // first chunk, and after a guard-path chunk; otherwise the previous
        // chunk step wrote them)
        norm_partials(raw, smem);
        __syncthreads();
      }
      norms_ready = false;
      const int fl = prep(raw, smem, scale, pro, ea, clen, pa);   // wave-uniform flags
      if constexpr (!Cfg::SG) {   // the single-gate form has no guard
        if (lane_fresh() == 0) FL[w] = fl;
      }
      compiler_fence();
      load_raw<LOAD_G>(raw, offs, q, k, v, g, beta, next, H, h, nlen);
      __syncthreads();                                           // B1
      int any = 0;
      if constexpr (!Cfg::SG) {
#pragma unroll
        for (int i = 0; i < NW; ++i) any |= FL[i];
      }
      if (!(any & 1)) {
        load_raw<LOAD_V>(raw, offs, q, k, v, g, beta, next, H, h, nlen);
        compiler_fence();
        f32x4 Y[4][NVT], O[4][NVT];
        // one instance per reference mode: the common chunk-start case
        // carries no block factors at all
        // the waves' modes are OR-ed: the strongest one present wins
        if (any & (KDA_MODE_SCALE << 1))
          middle<KDA_MODE_SCALE>(smem, S, Y, O);
        else if (any & (KDA_MODE_MASK << 1))
          middle<KDA_MODE_MASK>(smem, S, Y, O);
        else
          middle<KDA_MODE_CHUNK>(smem, S, Y, O);
        compiler_fence();
        load_raw<LOAD_Q | LOAD_K>(raw, offs, q, k, v, g, beta, next, H, h, nlen);
        __syncthreads();                                         // B2
        scan_step(smem, S, Y, O, out, row_base + c0, H, h, clen, raw, l2n);
        norms_ready = l2n;
      } else {
        // Some channel decays by more than 2^120 within one 16-token block
        // (log alpha averaging below about -5.2 over it, beyond the gate
        // transform's range), past what a block-start reference can scale:
        // the chunk runs the recurrence token by token on the same on-chip
        // state.  The next chunk's gates are already on their way; its q, k,
        // v follow here, so the loads in flight at the top of the loop are the
        // same on both paths.
        recurrent_chunk(S, q, k, v, g, beta, out, row_base + c0, H, h, clen, scale, pro, ea);
        load_raw<LOAD_Q | LOAD_K | LOAD_V>(raw, offs, q, k, v, g, beta, next, H, h, nlen);
        __syncthreads();                                         // LDS reuse
      }
    }
    if (S_final) {
      const int l = lane_fresh();
      const int n = l & 15, g4 = 4 * (l >> 4);
      float* Sf = S_final + chain * DK * DV + vw0 + n;
#pragma unroll
      for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
        for (int nt = 0; nt < NVT; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r) Sf[(16 * mt + g4 + r) * DV + 16 * nt] = S[mt][nt][r];
    }
  }
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS, 1) void chunk_fwd_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* S0, void* out,
    float* S_final, int T, int H, float scale, Prologue pro) {
  const int chain = blockIdx.x;   // b * H + h
  const int b = chain / H, h = chain % H;
  ChunkKernel<Cfg>::run(q, k, v, g, beta, S0, out, S_final, (size_t)b * T, T, H, h,
                        (size_t)chain, scale, pro);
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS, 1) void chunk_fwd_varlen_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* S0, void* out,
    float* S_final, const int32_t* __restrict__ cu_seqlens, int N, int H, float scale,
    Prologue pro) {
  // Longest sequences first: workgroup b takes head b % H of the (b / H)-th
  // longest sequence (ties by index), so that with skewed lengths the long
  // chains start in the first wave of workgroups instead of setting the tail.
  // Each workgroup ranks the lengths itself, from an LDS copy (up to
  // KDA_LPT_MAX sequences; beyond that the order is the packed order).
  const int r = blockIdx.x / H, h = blockIdx.x % H;
  int n = r;
  if (N <= KDA_LPT_MAX) {
    extern __shared__ __attribute__((aligned(16))) char smem_[];
    int* lens = reinterpret_cast<int*>(smem_);
    int* sel = lens + KDA_LPT_MAX;
    for (int m = threadIdx.x; m < N; m += Cfg::NTHREADS) lens[m] = cu_seqlens[m + 1] - cu_seqlens[m];
    __syncthreads();
    for (int m = threadIdx.x; m < N; m += Cfg::NTHREADS) {
      const int lm = lens[m];
      int rank = 0;
      for (int j = 0; j < N; ++j) rank += (lens[j] > lm) || (lens[j] == lm && j < m);
      if (rank == r) *sel = m;
    }
    __syncthreads();
    n = *sel;
    __syncthreads();   // the LDS is the kernel's from here on
  }
  const int chain = n * H + h;
  const int b0 = cu_seqlens[n], b1 = cu_seqlens[n + 1];
  ChunkKernel<Cfg>::run(q, k, v, g, beta, S0, out, S_final, (size_t)b0, b1 - b0, H, h,
                        (size_t)chain, scale, pro);
}

// ============================================================ balanced packed schedule
// With one workgroup per (sequence, head) chain, a CU that receives two chains
// runs their sum: with skewed lengths the busiest CU can exceed the average by
// most of a chain whatever the order (16 sequences of U{1024..65536} tokens at
// 32 heads: 1,183 chunk steps on the busiest CU against 1,058 on average).
// Calls with more chains than the GPU holds at once (up to four times as
// many), packed or batched, therefore take McNaughton's wrap-around rule for
// preemptive scheduling on identical machines (R. McNaughton, "Scheduling
// with deadlines and loss functions", Management Science 6(1), 1959) when the
// caller gives a workspace:
//
// - the resident workgroups form M machines of H workgroups, one per head, so
//   that the heads of a sequence still read the same token rows side by side;
// - the sequences, counted in chunks (an empty one counts one), are laid end
//   to end and cut into M slices of T = max(ceil(total / M), longest) chunks;
// - a sequence that crosses the boundary between slices m and m + 1 is split:
//   machine m + 1 runs its first chunks as its first piece and hands the fp32
//   state over through the workspace; machine m runs the rest as its last
//   piece.  No sequence is longer than T, so the first piece ends no later
//   than the last one starts: the makespan is T chunk steps, the bound for
//   any division of the work.
//
// Chunks stay aligned to their sequence and the state crosses in fp32, so the
// results are bit-identical to the one-workgroup-per-chain kernel.  Each
// workgroup takes its place from a ticket counter, in the order workgroups
// actually start; a machine's workgroups wait only on tickets taken earlier,
// whose first piece waits on nothing, so every wait ends whatever order the
// hardware starts workgroups in.  A wait is bounded all the same: past
// KDA_SPLIT_SPIN polls (or the count in the environment variable
// KDA_SPLIT_SPIN_POLLS, which tests set to 0 to take this path) the workgroup
// recomputes the first piece itself.
struct SplitWs {
  static constexpr size_t OFF_TICKET = 0;                             // u32
  static constexpr size_t OFF_T = 8;                                  // i64 slice length
  static constexpr size_t OFF_TOTAL = 16;                             // i64 total chunks
  static constexpr size_t OFF_FLAGS = 256;                            // u32 per slot
  static constexpr size_t OFF_PRE = OFF_FLAGS + KDA_SPLIT_MAX_WG * 4;  // i64 [N + 1]
  __host__ __device__ static size_t off_state(int N) { return (OFF_PRE + (size_t)(N + 1) * 8 + 255) / 256 * 256; }
  // handed-over states: slot m * H + h for the first piece on machine m >= 1;
  // a full slice holds the start of a sequence of index >= m, so m < N
  __host__ __device__ static int slots(int N, int H) {
    const long s = (long)N * H;
    return s < KDA_SPLIT_MAX_WG ? (int)s : KDA_SPLIT_MAX_WG;
  }
  __host__ __device__ static size_t bytes(int N, int H, int dk, int dv) {
    return off_state(N) + (size_t)slots(N, H) * dk * dv * 4;
  }
};

// Chunk counts per sequence -> prefix sums (i64), slice length and total; the
// ticket and every hand-over flag start at zero on each call.  cu == NULL: N
// sequences of Tfix tokens each (the batched layout).
__global__ __launch_bounds__(1024) void split_plan_kernel(const int32_t* __restrict__ cu, int N,
                                                          int Tfix, int C, int M, int nslots,
                                                          char* ws) {
  __shared__ long long wsum[16];
  __shared__ long long carry;
  __shared__ int umax;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  unsigned* flags = reinterpret_cast<unsigned*>(ws + SplitWs::OFF_FLAGS);
  long long* pre = reinterpret_cast<long long*>(ws + SplitWs::OFF_PRE);
  for (int i = tid; i < nslots; i += 1024) flags[i] = 0u;
  if (tid == 0) {
    *reinterpret_cast<unsigned*>(ws + SplitWs::OFF_TICKET) = 0u;
    pre[0] = 0;
    carry = 0;
    umax = 1;
  }
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    long long u = 0;
    if (n < N) {
      const int len = cu ? cu[n + 1] - cu[n] : Tfix;
      u = len > 0 ? (len + C - 1) / C : 1;
      atomicMax(&umax, (int)u);
    }
    long long x = u;   // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    long long off = carry;
    for (int i = 0; i < wv; ++i) off += wsum[i];
    if (n < N) pre[n + 1] = off + x;
    __syncthreads();
    if (tid == 0) {
      long long s = 0;
      for (int i = 0; i < 16; ++i) s += wsum[i];
      carry += s;
    }
    __syncthreads();
  }
  if (tid == 0) {
    const long long total = carry;
    long long T = (total + M - 1) / M;
    if (T < umax) T = umax;
    *reinterpret_cast<long long*>(ws + SplitWs::OFF_T) = T;
    *reinterpret_cast<long long*>(ws + SplitWs::OFF_TOTAL) = total;
  }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS, 1) void chunk_fwd_split_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* S0, void* out,
    float* S_final, const int32_t* __restrict__ cu, int N, int Tfix, int H, int M, int nslots,
    int spin, float scale, Prologue pro, char* ws) {
  extern __shared__ __attribute__((aligned(16))) char smem_[];
  LDS volatile int* sh = (LDS volatile int*)smem_;
  constexpr size_t SS = (size_t)Cfg::DK * Cfg::DV;
  constexpr int C = Cfg::C;
  if (threadIdx.x == 0)
    sh[0] = (int)atomicAdd(reinterpret_cast<unsigned*>(ws + SplitWs::OFF_TICKET), 1u);
  __syncthreads();
  const int id = sh[0];
  if (id >= M * H) return;
  // machine m = M - 1 - id / H: the first piece of machine m + 1, which
  // machine m's last piece waits for, belongs to a ticket H lower
  const int m = M - 1 - id / H, h = id % H;
  const long long T = *reinterpret_cast<const long long*>(ws + SplitWs::OFF_T);
  const long long total = *reinterpret_cast<const long long*>(ws + SplitWs::OFF_TOTAL);
  const long long* pre = reinterpret_cast<const long long*>(ws + SplitWs::OFF_PRE);
  unsigned* flags = reinterpret_cast<unsigned*>(ws + SplitWs::OFF_FLAGS);
  float* hand = reinterpret_cast<float*>(ws + SplitWs::off_state(N));
  long long x = (long long)m * T;
  const long long end = x + T < total ? x + T : total;
  while (x < end) {
    // the sequence holding chunk x of the concatenation: first n with pre[n + 1] > x
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (pre[mid + 1] > x) hi = mid;
      else lo = mid + 1;
    }
    const int n = lo;
    const long long s = pre[n], u = pre[n + 1] - s;
    // token rows of sequence n: packed from cu_seqlens, or n * Tfix batched
    const size_t b0 = cu ? (size_t)cu[n] : (size_t)n * Tfix;
    const int len = cu ? cu[n + 1] - cu[n] : Tfix;
    const size_t chain = (size_t)n * H + h;
    const float* sin = S0 ? S0 + chain * SS : nullptr;
    float* sout = S_final ? S_final + chain * SS : nullptr;
    long long c0 = 0, c1 = u;
    int post = -1, wait = -1;
    if (x > s) {   // begun in slice m - 1: the first chunks here, state handed on
      c1 = s + u - x;
      post = m * H + h;
      x = s + u;
    } else if (s + u > end) {   // runs past the slice: the rest is machine m + 1's first piece
      c0 = u - (end - s);
      wait = (m + 1) * H + h;
      x = end;
    } else {
      x = s + u;
    }
    if (post >= nslots || wait >= nslots) {   // outside the slots (excluded above): no split
      c0 = 0;
      c1 = u;
      post = wait = -1;
    }
    if (post >= 0) sout = hand + (size_t)post * SS;
    __syncthreads();   // the previous piece is done with the LDS
    if (wait >= 0) {
      if (threadIdx.x == 0) {
        int got = 0;
        for (int it = 0; it < spin && !got; ++it) {
          got = __hip_atomic_load(flags + wait, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != 0u;
          if (!got) __builtin_amdgcn_s_sleep(8);
        }
        sh[1] = got;
      }
      // thread 0's device-scope acquire, then the barrier, orders every
      // wave's reads of the handed-over state after the flag
      __syncthreads();
      const bool got = sh[1] != 0;
      if (got) sin = hand + (size_t)wait * SS;
      else c0 = 0;   // no hand-over in time: redo the first chunks here
      __syncthreads();
    }
    const long long r0 = (long long)C * c0;
    const long long r1 = (long long)C * c1 < len ? (long long)C * c1 : len;
    ChunkKernel<Cfg>::run(q, k, v, g, beta, sin, out, sout, b0 + (size_t)r0, (int)(r1 - r0), H,
                          h, 0, scale, pro);
    if (post >= 0) {
      // the barrier orders every wave's state stores before thread 0's
      // device-scope release (one write-back of this XCD's L2)
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_store(flags + post, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

size_t chunk_split_workspace_bytes(int n_seq, int H, int dk, int dv) {
  return SplitWs::bytes(n_seq, H, dk, dv);
}

// The poll limit of a hand-over wait: KDA_SPLIT_SPIN, or a non-negative count
// from the environment variable KDA_SPLIT_SPIN_POLLS (read on every call).
static int split_spin_polls() {
  const char* e = getenv("KDA_SPLIT_SPIN_POLLS");
  if (e && *e) {
    char* end = nullptr;
    const long v = strtol(e, &end, 10);
    if (end && *end == '\0' && v >= 0 && v <= KDA_SPLIT_SPIN) return (int)v;
  }
  return KDA_SPLIT_SPIN;
}

template <class Cfg>
static hipError_t launch_chunk_t(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* S0, void* out, float* S_final,
                                 const int32_t* cu, int n_seq, int T, int H, float scale,
                                 const Prologue& pro, void* ws, hipStream_t stream) {
  const int bytes = Cfg::LDS_TOTAL;
  if (ws) {
    // the balanced schedule when there are more chains than resident workgroups
    auto kern = chunk_fwd_split_kernel<Cfg>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    int dev = 0, cus = 0, occ = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, (const void*)kern, Cfg::NTHREADS, bytes);
    if (e != hipSuccess) return e;
    long P = (long)cus * (occ > 0 ? occ : 1);
    if (P > KDA_SPLIT_MAX_WG) P = KDA_SPLIT_MAX_WG;
    const int M = (int)(P / H);
    // up to 4 chains per workgroup: beyond that the hardware's dispatch of
    // whole chains, longest first, already evens the load and also absorbs
    // the CU-to-CU spread in speed, which a fixed split cannot
    const long chains = (long)n_seq * H;
    if (M >= 2 && chains > P && chains <= 4 * P) {
      const int nslots = SplitWs::slots(n_seq, H);
      hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(1024), 0, stream, cu, n_seq, T, Cfg::C,
                         M, nslots, (char*)ws);
      hipLaunchKernelGGL(kern, dim3(M * H), dim3(Cfg::NTHREADS), bytes, stream, q, k, v, g, beta,
                         S0, out, S_final, cu, n_seq, T, H, M, nslots, split_spin_polls(), scale,
                         pro, (char*)ws);
      return hipGetLastError();
    }
  }
  if (cu) {
    auto kern = chunk_fwd_varlen_kernel<Cfg>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_seq * H), dim3(Cfg::NTHREADS), bytes, stream, q, k, v, g,
                       beta, S0, out, S_final, cu, n_seq, H, scale, pro);
  } else {
    auto kern = chunk_fwd_kernel<Cfg>;
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(n_seq * H), dim3(Cfg::NTHREADS), bytes, stream, q, k, v, g,
                       beta, S0, out, S_final, T, H, scale, pro);
  }
  return hipGetLastError();
}

// ============================================================ chunk-parallel schedule
// For few (sequence, head) chains the one-workgroup-per-chain kernel leaves
// most CUs idle and its serial chunk chain sets the time.  This schedule
// follows the three-stage structure of "Kimi Unveils Delta Attention and K3
// Architecture Updates", section 6.6 (per-chunk WY factors, one inter-chunk
// state scan, outputs of all chunks in parallel), with the factors of section
// 6.3/6.4 written out in the key-by-value orientation:
//
//   W = (I + R)^{-1} Diag(beta) KG          U = (I + R)^{-1} Diag(beta) V
//   E_c = U - W S_c                         (the resolved errors of 6.3)
//   S_{c+1} = Diag(Gamma_L) S_c + K_end^T E_c,   K_end = Gamma_L * KI (6.4)
//   O_c = QG S_c + Aqk E_c                  (6.5)
//
// Stage A (chunk_intra_kernel, one workgroup per (chunk, head), all chunks at
// once) forms everything that does not depend on the state; stage B
// (chunk_scan_kernel, one workgroup per (chain, 16 value columns)) runs the
// only serial loop, two 128-deep products per chunk, in one wave, while its
// second wave forms each chunk's outputs from the state and errors the first
// hands over through the LDS.  Every factor goes through the workspace as
// bf16 MFMA fragments in the exact lane order its consumer reads, one 16-byte
// load per lane per fragment.  A chunk with a 16-token block that decays
// below 2^KDA_BLOCK_LOG2_MIN in some channel (the fused kernel's guard) is
// flagged by stage A and recomputed token by token by stage B.
template <class Cfg>
struct ParLayout {
  static constexpr int DK = Cfg::DK, DV = Cfg::DV;
  static constexpr int NKS = DK / 32, MTK = DK / 16, NVS = DV / 16;
  static constexpr int FR = 64 * 16;                          // one fragment, 64 lanes
  static constexpr int OFF_W = 0;                             // -W   [I 4][ks]
  static constexpr int OFF_QG = OFF_W + 4 * NKS * FR;         // QG   [I 4][ks]
  static constexpr int OFF_KE = OFF_QG + 4 * NKS * FR;        // -K_end^T [mt][kt 2]
  static constexpr int OFF_AQ = OFF_KE + MTK * 2 * FR;        // -Aqk [I 4][kt 2]
  static constexpr int OFF_U = OFF_AQ + 4 * 2 * FR;           // U    [vs][I 4][lane] 8 B
  static constexpr int OFF_GL = OFF_U + NVS * 4 * 64 * 8;     // Gamma_L [DK] fp32
  static constexpr int PER_CHUNK = OFF_GL + DK * 4;
  static_assert(PER_CHUNK % 256 == 0, "chunk records stay 256-byte aligned");
  // bytes of workspace for n chunk-heads: the records, then one int flag each
  static size_t bytes(size_t n) { return n * PER_CHUNK + ((n * 4 + 255) / 256) * 256; }
};

// Where the chunk-parallel records come from.  Batched (cu == NULL): chain
// b * H + h has NC chunks of the sequence at rows b * T, records chain * NC +
// c.  Packed: the chunk prefix sums pre[] of the balanced schedule's plan
// (split_plan_kernel; an empty sequence counts one chunk, of no tokens, which
// leaves its state as it is), the records of sequence n head-major from
// H * pre[n].
struct ParTable {
  const int32_t* cu;
  const long long* pre;
  int T, H, NC, C;
  // chain -> first record, chunks, first token row, tokens
  __device__ __forceinline__ void chain(int ch, long long& rec0, int& nc, size_t& row0,
                                        int& len) const {
    const int n = ch / H, h = ch % H;
    if (cu) {
      const long long p0 = pre[n];
      nc = (int)(pre[n + 1] - p0);
      rec0 = (long long)H * p0 + (long long)h * nc;
      row0 = (size_t)cu[n];
      len = cu[n + 1] - cu[n];
    } else {
      nc = NC;
      rec0 = (long long)ch * NC;
      row0 = (size_t)n * T;
      len = T;
    }
  }
  // record -> first token row of its chunk, head, tokens (0 past the end)
  __device__ __forceinline__ void record(long long idx, int N, size_t& row0, int& h,
                                         int& clen) const {
    if (cu) {
      int lo = 0, hi = N - 1;   // the sequence: first n with H * pre[n + 1] > idx
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((long long)H * pre[mid + 1] > idx) hi = mid;
        else lo = mid + 1;
      }
      const long long p0 = pre[lo];
      const int nc = (int)(pre[lo + 1] - p0);
      const long long r = idx - (long long)H * p0;
      h = (int)(r / nc);
      const int c = (int)(r % nc);
      const int len = cu[lo + 1] - cu[lo];
      row0 = (size_t)cu[lo] + (size_t)c * C;
      clen = max(0, min(C, len - c * C));
    } else {
      const int chain = (int)(idx / NC), c = (int)(idx % NC);
      h = chain % H;
      row0 = (size_t)(chain / H) * T + (size_t)c * C;
      clen = min(C, T - c * C);
    }
  }
};

template <class Cfg>
struct ParKernel {
  typedef ChunkKernel<Cfg> K;
  typedef ParLayout<Cfg> L;
  typedef typename Cfg::Op Op;
  typedef typename Cfg::T T;
  typedef typename Cfg::Io Io;
  static constexpr int C = Cfg::C, DK = Cfg::DK, DV = Cfg::DV, NW = Cfg::NW;
  static constexpr int NKS = Cfg::NKS, MTK = Cfg::MTK;
  static_assert(NW == 8 && DK == 128 && DV == 128 && Op::PERMUTED, "bf16 128x128 only");

  static __device__ __forceinline__ void st16(char* p, typename Op::F32 f) {
    *reinterpret_cast<u32x4*>(p) = __builtin_bit_cast(u32x4, __builtin_shufflevector(f.lo, f.hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  static __device__ __forceinline__ typename Op::F32 ld16(const char* p) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(p);
    const i16x8 v = __builtin_bit_cast(i16x8, w);
    return typename Op::F32{__builtin_shufflevector(v, v, 0, 1, 2, 3), __builtin_shufflevector(v, v, 4, 5, 6, 7)};
  }
  static __device__ __forceinline__ typename Op::F16 neg16(typename Op::F16 f) {
    return __builtin_bit_cast(typename Op::F16, __builtin_bit_cast(u32x2, f) ^ u32x2{0x80008000u, 0x80008000u});
  }

  // The state-independent tiles and inverses (the fused kernel's middle
  // interval without its state products).
  template <int MODE>
  static __device__ __forceinline__ void tiles(LDS char* smem) {
    switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
      case 0: K::template tile_qk<MODE>(smem, 0, 0); K::template invert_diag<0>(smem); break;
      case 1: K::template tile_qk<MODE>(smem, 1, 1); K::template invert_diag<1>(smem); break;
      case 2: K::template tile_qk<MODE>(smem, 2, 2); K::template invert_diag<2>(smem); break;
      case 3: K::template tile_qk<MODE>(smem, 3, 3); K::template invert_diag<3>(smem); break;
      case 4: K::template tile_qk<MODE>(smem, 1, 0); K::template tile_qk<MODE>(smem, 3, 2); break;
      case 5: K::template tile_qk<MODE>(smem, 2, 0); K::template tile_qk<MODE>(smem, 2, 1); break;
      case 6: K::template tile_qk<MODE>(smem, 3, 0); break;
      default: K::template tile_qk<MODE>(smem, 3, 1); break;
    }
  }

  // X = (I + R)^{-1} Y by 16-token blocks for this wave's two 16-column tiles:
  // waves 0-3 take Y = Diag(beta) k Gamma (key columns 32w ..; for channels
  // referenced to the block start the KG buffer holds k Pi, so block I takes
  // P_I on each key column, 1 for the others), so X = W; waves 4-7 take
  // Y = Diag(beta) (-V) (value columns 32(w-4) ..), so X = -U.
  // -W goes back into the KG buffer (the wave's own columns, which only it
  // reads from here on); U goes straight to the workspace in the
  // accumulator layout stage B starts E from.
  static __device__ __forceinline__ void wy(LDS char* smem, char* rec) {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const int n = l & 15, g = l >> 4;
    LDS T* KG = (LDS T*)(smem + Cfg::OFF_KG);
    const LDS T* BV = (const LDS T*)(smem + Cfg::OFF_BV);
    const LDS T* RR = (const LDS T*)(smem + Cfg::OFF_RT);
    const LDS T* TD = (const LDS T*)(smem + Cfg::OFF_TD);
    const LDS float* BT = (const LDS float*)(smem + Cfg::OFF_BT);
    const LDS float* DP = (const LDS float*)(smem + Cfg::OFF_DP);
    const bool keys = w < 4;
    const int c0 = 32 * (w & 3);
    f32x4 Y[4][2];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      const f32x4 b = *lds_ptr<const f32x4>(BT + 16 * I + 4 * g);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const typename Op::F16 f = keys ? Op::ld16_trp(l, KG, Cfg::LD_K, 16 * I, Op::perm_pos(c0 + 16 * nt))
                                        : Op::ld16_tr(l, BV, Cfg::LD_V, 16 * I, c0 + 16 * nt);
        const float pf = (keys && I > 0) ? DP[I * DK + frag_pos(c0 + 16 * nt + n)] : 1.f;
        Y[I][nt] = Op::unpack(f) * (b * pf);
      }
    }
    typename Op::F16 XP[4][2];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      if (I > 0) {
        f32x4 Z[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int J = 0; J < I; ++J) {
          const typename Op::F16 a = Op::ld16_rm(l, RR, Cfg::LD_RR, 16 * I, 16 * J);   // -R_IJ
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) Z[nt] = Op::mma16(a, XP[J][nt], Z[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) Y[I][nt] += Z[nt];
      }
      const typename Op::F16 a = Op::ld16_tr(l, TD + I * 256, 16, 0, 0);   // T_II
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        XP[I][nt] = Op::pack(Op::mma16(a, Op::pack(Y[I][nt]), z));
      }
    }
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if (keys) {
          // -W[16I + 4g + r][c0 + 16nt + n] into the (permuted) KG rows
          const u32x2 wv = __builtin_bit_cast(u32x2, neg16(XP[I][nt]));
          const int col = Op::perm_pos(c0 + 16 * nt + n);
          LDS uint16_t* p = (LDS uint16_t*)(KG) + (16 * I + 4 * g) * Cfg::LD_K + col;
          p[0] = (uint16_t)(wv[0] & 0xffffu);
          p[Cfg::LD_K] = (uint16_t)(wv[0] >> 16);
          p[2 * Cfg::LD_K] = (uint16_t)(wv[1] & 0xffffu);
          p[3 * Cfg::LD_K] = (uint16_t)(wv[1] >> 16);
        } else {
          // U = -X: value tile vs = (c0 + 16nt) / 16, token block I, this lane
          const int vs = (c0 + 16 * nt) / 16;
          *reinterpret_cast<u32x2*>(rec + L::OFF_U + ((vs * 4 + I) * 64 + l) * 8) =
              __builtin_bit_cast(u32x2, neg16(XP[I][nt]));
        }
      }
  }

  // The remaining factors to the workspace, each as the fragments their
  // consumers read: -W and QG = s q Gamma (rows = tokens, k = keys; block I
  // takes P_I on each block-referenced channel), -K_end^T
  // (rows = keys, k = tokens), -Aqk (rows = tokens, k = tokens), Gamma_L.
  static __device__ __forceinline__ void write_factors(LDS char* smem, char* rec) {
    const int w = threadIdx.x >> 6, l = lane_fresh();
    const LDS T* KG = (const LDS T*)(smem + Cfg::OFF_KG);   // now -W
    const LDS T* QG = (const LDS T*)(smem + Cfg::OFF_QG);
    const LDS T* KIT = (const LDS T*)(smem + Cfg::OFF_KT);
    const LDS T* AQ = (const LDS T*)(smem + Cfg::OFF_AQ);
    const LDS float* GL = (const LDS float*)(smem + Cfg::OFF_GL);
    const LDS float* DP = (const LDS float*)(smem + Cfg::OFF_DP);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int f = 2 * w + j;                  // 0 .. 15
      const int I = f / NKS, ks = f % NKS;
      st16(rec + L::OFF_W + f * L::FR + l * 16, Op::ld32_rmp(l, KG, Cfg::LD_K, 16 * I, 32 * ks));
      typename Op::F32 qf = Op::ld32_rmp(l, QG, Cfg::LD_K, 16 * I, 32 * ks);
      if (I > 0) {
        const LDS float* P = DP + I * DK + 32 * ks + 8 * (l >> 4);
        qf.lo = Op::pack(Op::unpack(qf.lo) * *lds_ptr<const f32x4>(P));
        qf.hi = Op::pack(Op::unpack(qf.hi) * *lds_ptr<const f32x4>(P + 4));
      }
      st16(rec + L::OFF_QG + f * L::FR + l * 16, qf);
      const int mt = f / 2, kt = f % 2;         // KIT holds -K_end key-major
      st16(rec + L::OFF_KE + f * L::FR + l * 16, Op::ld32_rmp(l, KIT, Cfg::LD_KT, 16 * mt, 32 * kt));
    }
    st16(rec + L::OFF_AQ + w * L::FR + l * 16, Op::ld32_rmp(l, AQ, Cfg::LD_AQ, 16 * (w / 2), 32 * (w % 2)));
    if (w == 0 && l < DK / 4)
      *reinterpret_cast<f32x4*>(rec + L::OFF_GL + 16 * l) = *lds_ptr<const f32x4>(GL + 4 * l);
  }
};

// Stage A: persistent workgroups, each taking (chain, chunk) records idx =
// chain * NC + chunk in steps of the grid size; the next record's raw inputs
// are loaded in three batches while the current one is formed.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NTHREADS, 1) void chunk_intra_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, char* __restrict__ ws,
    int* __restrict__ flags, ParTable tab, int N, long long total_host,
    const long long* __restrict__ total_dev, float scale) {
  typedef ChunkKernel<Cfg> K;
  typedef ParLayout<Cfg> L;
  typedef ParKernel<Cfg> P;
  typedef typename Cfg::Op Op;
  typedef typename Cfg::T OpT;
  extern __shared__ __attribute__((aligned(16))) char smem_[];
  LDS char* smem = (LDS char*)smem_;
  const int H = tab.H;
  // records: known on the host when batched, H times the plan's chunk total when packed
  const long long total = total_dev ? (long long)H * *total_dev : total_host;
  {
    LDS OpT* AQ = (LDS OpT*)(smem + Cfg::OFF_AQ);   // tiles above the diagonal stay zero
    for (int i = threadIdx.x; i < Cfg::C * Cfg::LD_AQ; i += Cfg::NTHREADS) AQ[i] = Op::cvt(0.f);
  }
  // record idx -> first token row, head, tokens
  auto where = [&](long long idx, size_t& row0, int& h, int& clen) {
    tab.record(idx, N, row0, h, clen);
  };
  const typename K::Offsets offs = K::lane_offsets(H);
  const typename K::PrepAddr pa = K::prep_addr();
  const Prologue pro{0u, nullptr, nullptr};
  LDS int* FL = (LDS int*)(smem + Cfg::OFF_FL);
  const int w = threadIdx.x >> 6;
  typename K::Raw raw;
  size_t row0 = 0;
  int h = 0, clen = 0;
  if (blockIdx.x < total) where(blockIdx.x, row0, h, clen);
  K::template load_raw<K::LOAD_ALL>(raw, offs, q, k, v, g, beta, row0, H, h, clen);
  for (long long idx = blockIdx.x; idx < total; idx += gridDim.x) {
    // the next record (an empty range after the last: nothing is read)
    const long long nidx = idx + gridDim.x;
    size_t nrow0 = row0;
    int nh = h, nlen = 0;
    if (nidx < total) where(nidx, nrow0, nh, nlen);
    const int fl = K::prep(raw, smem, scale, pro, 1.f, clen, pa);   // wave-uniform flags
    if (lane_fresh() == 0) FL[w] = fl;
    compiler_fence();
    K::template load_raw<K::LOAD_G>(raw, offs, q, k, v, g, beta, nrow0, H, nh, nlen);
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int i = 0; i < Cfg::NW; ++i) any |= FL[i];
    const int any_bad = any & 1;
    if (threadIdx.x == 0) flags[idx] = any_bad;
    // a flagged chunk is redone token by token by stage B
    K::template load_raw<K::LOAD_V>(raw, offs, q, k, v, g, beta, nrow0, H, nh, nlen);
    compiler_fence();
    if (!any_bad) {
      // the waves' modes are OR-ed: the strongest one present wins
      if (any & (KDA_MODE_SCALE << 1))
        P::template tiles<KDA_MODE_SCALE>(smem);
      else if (any & (KDA_MODE_MASK << 1))
        P::template tiles<KDA_MODE_MASK>(smem);
      else
        P::template tiles<KDA_MODE_CHUNK>(smem);
    }
    compiler_fence();
    __syncthreads();
    K::template load_raw<K::LOAD_Q | K::LOAD_K>(raw, offs, q, k, v, g, beta, nrow0, H, nh, nlen);
    char* rec = ws + (size_t)idx * L::PER_CHUNK;
    if (!any_bad) P::wy(smem, rec);
    __syncthreads();
    if (!any_bad) P::write_factors(smem, rec);
    __syncthreads();   // the LDS is free for the next record's prep
    row0 = nrow0;
    h = nh;
    clen = nlen;
  }
}

// Stage B: one workgroup per (chain, 16 value columns), two waves.
// Wave 0 scans the state: the fragments of chunk c + 1 are loaded while chunk
// c is computed (-W right after its last use, -K_end, U and Gamma_L after the
// state update).  It puts S_c and -E_c, as the bf16 fragments it multiplies
// anyway, into one of two LDS slots and meets wave 1 at one barrier per chunk.
// Wave 1 forms O_c^T = S_c^T QG^T + (-E_c)^T (-Aqk)^T from that slot, its
// own factors a chunk ahead, and writes 4 consecutive values of a token per
// lane.  Slot c & 1 is written again only for chunk c + 2, after the barrier
// of chunk c + 1, which wave 1 reaches once it has read chunk c.
template <class Cfg>
__global__ __launch_bounds__(128, 1) void chunk_scan_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* S0, void* out,
    float* S_final, char* __restrict__ ws, const int* __restrict__ flags, ParTable tab,
    int n_chains, float scale) {
  // flags: stage A's per-chunk flags, read-only here (scalar loads: a vector
  // load would make each step wait for every prefetched factor)
  typedef ChunkKernel<Cfg> K;
  typedef ParLayout<Cfg> L;
  typedef ParKernel<Cfg> P;
  typedef typename Cfg::Op Op;
  typedef typename Cfg::Io Io;
  typedef typename Op::F32 Frag;
  constexpr int MTK = Cfg::MTK, NKS = Cfg::NKS, DK = Cfg::DK, DV = Cfg::DV;
  constexpr int SLOT = (NKS + 2) * L::FR;   // S_c [ks][lane], then -E_c [kt 2][lane]
  __shared__ __attribute__((aligned(16))) char ring_[2 * SLOT];
  LDS char* ring = (LDS char*)ring_;
  // Workgroups are dealt to the 8 XCDs round robin (block i on XCD i % 8):
  // the NVS slices of one chain go to one XCD, so that they share its L2 for
  // the chain's factors.  Blocks past the last chain have nothing to do.
  static_assert(L::NVS == 8, "eight value slices per chain");
  const int xcd = blockIdx.x % 8, r = blockIdx.x / 8;
  const int chain = (r / L::NVS) * 8 + xcd, vs = r % L::NVS;
  if (chain >= n_chains) return;
  const int H = tab.H, h = chain % H;
  long long rec0;
  int NC, T;
  size_t row_base;
  tab.chain(chain, rec0, NC, row_base, T);   // the chain's records and token rows
  const int w = threadIdx.x >> 6;
  const int l = lane_fresh();
  const int n = l & 15, g4 = 4 * (l >> 4);
  auto rec_of = [&](int c) { return ws + (size_t)(rec0 + (c < NC ? c : NC - 1)) * L::PER_CHUNK; };
  auto st_slot = [&](int off, Frag f) {
    *(LDS u32x4*)(ring + off + l * 16) =
        __builtin_bit_cast(u32x4, __builtin_shufflevector(f.lo, f.hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto ld_slot = [&](int off) {
    const u32x4 x = *(const LDS u32x4*)(ring + off + l * 16);
    const i16x8 y = __builtin_bit_cast(i16x8, x);
    return Frag{__builtin_shufflevector(y, y, 0, 1, 2, 3), __builtin_shufflevector(y, y, 4, 5, 6, 7)};
  };
  // Chunks stage A flagged are redone token by token by wave 0, which also
  // writes their outputs; a chain without any runs loops with no branch inside.
  int any_flag = 0;
  for (int c = 0; c < NC; ++c) any_flag |= flags[rec0 + c];

  if (w == 1) {
    // ---- wave 1: the outputs
    struct OFac {
      Frag Q[4][NKS], A[4][2];
    };
    auto load_o = [&](OFac& f, const char* rec) {
#pragma unroll
      for (int i = 0; i < 4 * NKS; ++i) f.Q[i / NKS][i % NKS] = P::ld16(rec + L::OFF_QG + i * L::FR + l * 16);
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int kt = 0; kt <= I / 2; ++kt) f.A[I][kt] = P::ld16(rec + L::OFF_AQ + (I * 2 + kt) * L::FR + l * 16);
    };
    auto out_step = [&](int c, OFac& f, int pf) {
      __syncthreads();   // chunk c's S_c and -E_c are in slot c & 1
      const int so = (c & 1) * SLOT;
      Frag SB[NKS], EB[2];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) SB[ks] = ld_slot(so + ks * L::FR);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) EB[kt] = ld_slot(so + (NKS + kt) * L::FR);
      const int clen = min(Cfg::C, T - c * Cfg::C);
      f32x4 o[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        o[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) o[I] = Op::mma32(SB[ks], f.Q[I][ks], o[I]);
#pragma unroll
        for (int kt = 0; kt <= I / 2; ++kt) o[I] = Op::mma32(EB[kt], f.A[I][kt], o[I]);
      }
      if (pf >= 0) load_o(f, rec_of(pf));
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int t = 16 * I + (l & 15);
        if (t < clen) {
          const size_t row = (row_base + (size_t)c * Cfg::C + t) * H + h;
          Io::store4(out, row * DV + 16 * vs + 4 * (l >> 4), o[I]);
        }
      }
    };
    if (!any_flag) {
      OFac fa, fb;
      load_o(fa, rec_of(0));
      load_o(fb, rec_of(1));
      int c = 0;
      for (; c + 1 < NC; c += 2) {
        out_step(c, fa, c + 2);
        out_step(c + 1, fb, c + 3);
      }
      if (c < NC) out_step(c, fa, -1);
    } else {
      OFac fa;
      for (int c = 0; c < NC; ++c) {
        if (flags[rec0 + c]) {
          __syncthreads();   // written token by token by wave 0
        } else {
          load_o(fa, rec_of(c));
          out_step(c, fa, -1);
        }
      }
    }
    return;
  }

  // ---- wave 0: the state scan
  f32x4 S[MTK][1];
#pragma unroll
  for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[mt][0][r] = S0 ? S0[((size_t)chain * DK + 16 * mt + g4 + r) * DV + 16 * vs + n] : 0.f;
  // The factors of one chunk in registers.
  struct Fac {
    Frag W[4][NKS], K[MTK][2];
    u32x2 U[4];
    f32x4 G[MTK];
  };
  auto load_w = [&](Fac& f, const char* rec) {
#pragma unroll
    for (int i = 0; i < 4 * NKS; ++i) f.W[i / NKS][i % NKS] = P::ld16(rec + L::OFF_W + i * L::FR + l * 16);
  };
  // in the order of use: U (end of the E products), Gamma_L, -K_end (state update)
  auto load_rest = [&](Fac& f, const char* rec) {
#pragma unroll
    for (int I = 0; I < 4; ++I) f.U[I] = *reinterpret_cast<const u32x2*>(rec + L::OFF_U + ((vs * 4 + I) * 64 + l) * 8);
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt) f.G[mt] = *reinterpret_cast<const f32x4*>(rec + L::OFF_GL + (16 * mt + g4) * 4);
#pragma unroll
    for (int i = 0; i < 2 * MTK; ++i) f.K[i / 2][i % 2] = P::ld16(rec + L::OFF_KE + i * L::FR + l * 16);
  };
  // One step of the scan on chunk c from the factors in f; with pf >= 0 the
  // factors of chunk pf are loaded into f behind it (-W after its last use,
  // the rest after the state update).
  auto step = [&](int c, Fac& f, int pf) {
    const int so = (c & 1) * SLOT;
    // S_c as 32-deep operands over keys (also wave 1's A operand)
    Frag SB[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      SB[ks] = Frag{Op::pack(S[2 * ks][0]), Op::pack(S[2 * ks + 1][0])};
      st_slot(so + ks * L::FR, SB[ks]);
    }
    // E = U + (-W) S_c
    f32x4 E[4];
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      E[I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) E[I] = Op::mma32(f.W[I][ks], SB[ks], E[I]);
      E[I] += Op::unpack(__builtin_bit_cast(typename Op::F16, f.U[I]));
    }
    if (pf >= 0) load_w(f, rec_of(pf));
    // -E as 32-deep operands over tokens
    Frag EB[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      EB[kt] = Frag{Op::pack(-E[2 * kt]), Op::pack(-E[2 * kt + 1])};
      st_slot(so + (NKS + kt) * L::FR, EB[kt]);
    }
    __syncthreads();   // slot c & 1 to wave 1
    // S <- Diag(Gamma_L) S + (-K_end)^T (-E)
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt) {
      f32x4 s = S[mt][0] * f.G[mt];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s = Op::mma32(f.K[mt][kt], EB[kt], s);
      S[mt][0] = s;
    }
    if (pf >= 0) load_rest(f, rec_of(pf));
  };
  if (!any_flag) {
    // two chunks of factors in flight (so that the loads stay where they are
    // issued, a chunk ahead of their use)
    Fac fa, fb;
    load_w(fa, rec_of(0));
    load_rest(fa, rec_of(0));
    load_w(fb, rec_of(1));
    load_rest(fb, rec_of(1));
    int c = 0;
    for (; c + 1 < NC; c += 2) {
      step(c, fa, c + 2);
      step(c + 1, fb, c + 3);
    }
    if (c < NC) step(c, fa, -1);
  } else {
    // (rare) without prefetching
    Fac fa;
    for (int c = 0; c < NC; ++c) {
      if (flags[rec0 + c]) {
        // outside the chunk-start reference's range: the recurrence token by token
        const Prologue pro{0u, nullptr, nullptr};
        K::recurrent_chunk(S, q, k, v, g, beta, out, row_base + (size_t)c * Cfg::C, H, h,
                           min(Cfg::C, T - c * Cfg::C), scale, pro, 1.f, 16 * vs);
        __syncthreads();   // wave 1 skips this chunk
      } else {
        load_w(fa, rec_of(c));
        load_rest(fa, rec_of(c));
        step(c, fa, -1);
      }
    }
  }
  if (S_final) {
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S_final[((size_t)chain * DK + 16 * mt + g4 + r) * DV + 16 * vs + n] = S[mt][0][r];
  }
}

// The schedule by shape: bf16 128x128 calls of few, long chains take the
// chunk-parallel stages (the state chain of each sequence is then 128-deep
// products only); everything else the one-workgroup-per-chain kernel.
size_t chunk_par_workspace_bytes(int n_seq, int T, int H) {
  typedef ChunkCfg<128, 128, IoBf16, OpBf16, 8, false, false> Cfg;
  const size_t NC = (size_t)(T + Cfg::C - 1) / Cfg::C;
  return ParLayout<Cfg>::bytes((size_t)n_seq * H * NC);
}

// Packed: the chunk table (the balanced schedule's plan region), then records
// for at most H * (ceil(T_total / C) + N) chunks (each sequence's last chunk
// may be partial; an empty sequence takes one record).
static size_t par_varlen_records(int N, int T_total, int H) {
  const size_t C = 64;
  return (size_t)H * (((size_t)T_total + C - 1) / C + (size_t)N);
}

size_t chunk_par_varlen_workspace_bytes(int N, int T_total, int H) {
  typedef ChunkCfg<128, 128, IoBf16, OpBf16, 8, false, false> Cfg;
  static_assert(Cfg::C == 64, "chunk");
  return SplitWs::off_state(N) + ParLayout<Cfg>::bytes(par_varlen_records(N, T_total, H));
}

bool chunk_par_selected(int n_seq, int T, int H, int dk, int dv, bool bf16) {
  return bf16 && dk == 128 && dv == 128 && n_seq > 0 && (long)n_seq * H <= KDA_PAR_MAX_CHAINS &&
         T >= KDA_PAR_MIN_T && chunk_par_workspace_bytes(n_seq, T, H) <= KDA_PAR_MAX_WS;
}

// packed: the same few chains, at least KDA_PAR_MIN_T tokens per sequence on average
bool chunk_par_varlen_selected(int N, int T_total, int H, int dk, int dv, bool bf16) {
  return bf16 && dk == 128 && dv == 128 && N > 0 && (long)N * H <= KDA_PAR_MAX_CHAINS &&
         (long)T_total >= (long)KDA_PAR_MIN_T * N &&
         chunk_par_varlen_workspace_bytes(N, T_total, H) <= KDA_PAR_MAX_WS;
}

// cu == NULL: n_seq sequences of T tokens (batched); otherwise packed, T = T_total
hipError_t launch_chunk_par(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* S0, void* out, float* S_final,
                            const int32_t* cu, int n_seq, int T, int H, float scale, void* ws,
                            hipStream_t stream) {
  typedef ChunkCfg<128, 128, IoBf16, OpBf16, 8, false, false> Cfg;
  typedef ParLayout<Cfg> L;
  const int NC = (T + Cfg::C - 1) / Cfg::C;
  const int chains = n_seq * H;
  const int bytes = Cfg::LDS_TOTAL;
  auto ka = chunk_intra_kernel<Cfg>;
  hipError_t e = hipFuncSetAttribute((const void*)ka, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  // one persistent workgroup per CU (the LDS holds one)
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  ParTable tab{cu, nullptr, T, H, NC, Cfg::C};
  char* rec = (char*)ws;
  size_t R;
  long long total_host = 0;
  const long long* total_dev = nullptr;
  int grid_a;
  if (cu) {
    // the chunk table: chunks per sequence as prefix sums (the plan kernel,
    // one machine; its slice length goes unused)
    hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(1024), 0, stream, cu, n_seq, T, Cfg::C, 1,
                       0, (char*)ws);
    tab.pre = reinterpret_cast<const long long*>((char*)ws + SplitWs::OFF_PRE);
    total_dev = reinterpret_cast<const long long*>((char*)ws + SplitWs::OFF_TOTAL);
    rec = (char*)ws + SplitWs::off_state(n_seq);
    R = par_varlen_records(n_seq, T, H);
    grid_a = cus;   // workgroups past the last record exit at once
  } else {
    R = (size_t)chains * NC;
    total_host = (long long)R;
    grid_a = total_host < cus ? (int)total_host : cus;
  }
  int* flags = reinterpret_cast<int*>(rec + R * L::PER_CHUNK);
  hipLaunchKernelGGL(ka, dim3(grid_a), dim3(Cfg::NTHREADS), bytes, stream, q, k, v, g, beta, rec,
                     flags, tab, n_seq, total_host, total_dev, scale);
  const int grid_b = (chains + 7) / 8 * 8 * L::NVS;
  hipLaunchKernelGGL(chunk_scan_kernel<Cfg>, dim3(grid_b), dim3(128), 0, stream, q, k, v, g, beta,
                     S0, out, S_final, rec, flags, tab, chains, scale);
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
                        float scale, bool bf16, bool scalar_gate, const Prologue& pro, void* ws,
                        hipStream_t stream) {
  const bool fu = pro.flags != 0;
#define KDA_CH1(DK, DV, IO, OP, NWV, SG, FU)                                                 \
  return launch_chunk_t<ChunkCfg<DK, DV, IO, OP, NWV, SG, FU>>(                              \
      q, k, v, g, beta, S0, out, S_final, cu_seqlens, n_seq, T, H, scale, pro, ws, stream);
#define KDA_CH(DK, DV, IO, OP, NWV)                                       \
  if (scalar_gate) {                                                      \
    if (fu) { KDA_CH1(DK, DV, IO, OP, NWV, true, true) }                  \
    KDA_CH1(DK, DV, IO, OP, NWV, true, false)                             \
  }                                                                       \
  if (fu) { KDA_CH1(DK, DV, IO, OP, NWV, false, true) }                   \
  KDA_CH1(DK, DV, IO, OP, NWV, false, false)
  // d_v = 128 runs 8 waves (two per SIMD, 16 value columns each); d_v = 64
  // keeps 4 (value tiles are 16 columns wide).
  if (bf16) {
    if (dk == 128 && dv == 128) { KDA_CH(128, 128, IoBf16, OpBf16, 8) }
    if (dk == 128 && dv == 64) { KDA_CH(128, 64, IoBf16, OpBf16, 4) }
    if (dk == 64 && dv == 128) { KDA_CH(64, 128, IoBf16, OpBf16, 8) }
    if (dk == 64 && dv == 64) { KDA_CH(64, 64, IoBf16, OpBf16, 4) }
  } else {
    if (dk == 64 && dv == 64) { KDA_CH(64, 64, IoF32, OpF32, 4) }
  }
#undef KDA_CH
#undef KDA_CH1
  return hipErrorInvalidValue;
}

}  // namespace kda
