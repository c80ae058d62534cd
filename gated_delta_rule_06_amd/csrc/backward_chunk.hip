// backward_chunk.hip -- chunkwise backward on MFMA (bf16 I/O, d_k = d_v = 128).
//
// The gradients of the recurrence of "Kimi Unveils Delta Attention and K3
// Architecture Updates", section 4, taken through its chunkwise form (section
// 6, the training schedule): per chunk of C = 32 tokens with incoming state
// S_c, cumulative log decay b_i (inclusive prefix sum of g inside the chunk)
// and a per-channel reference r = b_15 (the chunk's middle),
//
//   QG = s Q e^{b-r}   KG = K e^{b-r}   KI = K e^{r-b}         (per element)
//   A   = strict_tril(KG KI^T)          Aqk = tril(QG KI^T)     (sections 6.3, 6.5)
//   T   = (I + Diag(beta) A)^{-1}       W = T Diag(beta) KG     U = T Diag(beta) V
//   S_m = Diag(e^r) S_c                 E = U - W S_m           (section 6.4)
//   O   = QG S_m + Aqk E                S_{c+1} = Diag(e^{b_L - r}) (S_m + KI^T E)
//
// Every product of a row factor and a column factor is e^{b_i - b_j}, so the
// chunk's algebra is that of section 6 exactly; the reference only keeps the
// stored factors within e^{+-76} when the chunk's two halves each decay by at
// most that much in every channel (log alpha above about -4.7 on average over
// 16 tokens, which covers the range (-5, 0) the pages give for K3's gates but
// for saturated runs).  A chain with a chunk beyond that is flagged and left to
// the token-by-token backward.
//
// Reverse mode, per chunk, given dS = dL/dS_{c+1} and dO (dS_m = Diag(e^{b_L-r}) dS):
//   dE  = KI dS_m + Aqk^T dO                 dS_c = Diag(e^r)(dS_m + QG^T dO - W^T dE)
//   dQG = dO S_m^T + dAqk KI,  dAqk = tril(dO E^T)
//   dW  = -dE S_m^T,  dY = T^T [dE | dW],  dV = beta dY_v,  dKG = beta dY_k + dA KI
//   dL  = -(dY_v U^T + dY_k W^T) (strict lower),  dA = Diag(beta) dL
//   dbeta_i = sum_j dL_ij A_ij + dY_v,i . V_i + dY_k,i . KG_i
//   dKI = dA^T KG + dAqk^T QG + E dS_m^T
//   dq = s e^{b-r} dQG,  dk = e^{b-r} dKG + e^{r-b} dKI
//   db = q dq + k (e^{b-r} dKG - e^{r-b} dKI),  plus sum_v dS S_{c+1} on the last token
//   dlog_alpha_t = sum_{i >= t} db_i  (inside the chunk)
// The loss does not depend on r (it cancels in every product), so r is held
// constant in the derivative.  The kernel forms dlog alpha in an equal order
// that cancels in fp32: db from the same bf16 factors the products used
// (QG dQG + KG dKG - KI dKI), the K_end part of dKI (E dS_m^T) as a sum over
// the tokens before t, and the incoming state's decay (sum_v dS_m S_m) on
// every token.
//
// Mapping (one workgroup of 8 waves per (sequence, head) chain):
//  * a forward sweep carries S in fp32 registers and stores each chunk's S_c
//    to the workspace as bf16 (the lanes' own order, 512 contiguous bytes per
//    wave and tile); the reverse sweep reads S_c back and carries dS in fp32;
//  * wave w owns value columns [16w, 16w+16) of S, dS, U, E, dE and dY_v, and
//    key channels [16w, 16w+16) of dQG, dW, dY_k, dKG and dKI; a lane's prep
//    elements (tokens 4g + r and 16 + 4g + r, channel 16w + l%16, g = lane/16)
//    are exactly its accumulator elements of the latter, so the epilogue needs
//    no exchange;
//  * the inputs load one chunk ahead as whole token rows (wave w takes tokens
//    4w .. 4w+3) and go through a shared [token][channel] staging area in
//    LDS, from which every wave takes its own columns with the transpose read;
//  * the in-chunk prefix sums (b) and the suffix sums of dlog alpha are
//    running sums in registers joined across lane groups by gfx950's permlane
//    swaps;
//  * operands go through LDS transposed ([channel][token]), the accumulator's
//    natural 8-byte store; contractions over tokens read rows, contractions
//    over channels use the gfx950 transpose read (ds_read_b64_tr_b16); S and
//    dS in registers serve as 32-deep operands with the k index relabelled
//    (two stacked 16-row accumulator tiles);
//  * T is formed in fp32: in the forward sweep the A tiles on one wave, handed
//    to the last, which solves the two 16x16 diagonal blocks by forward
//    substitution (a lane group each), then T_10 = -T_11 N_10 T_00 as MFMAs.
#include <stdlib.h>

#include "common.h"

namespace kda {

namespace {

#define LDS __attribute__((address_space(3)))

constexpr int BC = 32;          // tokens per chunk
constexpr int DD = 128;         // d_k = d_v
constexpr int NW = 8;           // waves
constexpr int NT = 64 * NW;     // threads
constexpr int LT = BC + 8;      // row length (bf16) of [channel][token] buffers: 80 bytes
constexpr int LR = DD + 8;      // row length (bf16) of the [value][channel] state buffer
constexpr int LA = BC + 4;      // row length (fp32) of A and T (16-byte rows)
constexpr float RANGE = 76.f;   // bound on |b_i - r| for the stored factors
constexpr int ST_DW = DD * DD / 2;     // dwords of one bf16 state
constexpr int SLOT_DW = ST_DW + 2 * BC * BC / 2;   // a chunk's workspace slot: S_c, T^T, (T Diag(beta))^T

// LDS layout (bytes)
constexpr int SZ_T = DD * LT * 2;      // [128][40] bf16
constexpr int SZ_S = BC * LT * 2;      // [32][40] bf16
constexpr int SZ_F = BC * LA * 4;      // [32][33] fp32
constexpr int O_QG = 0;
constexpr int O_KG = O_QG + SZ_T;
constexpr int O_KI = O_KG + SZ_T;
constexpr int O_V = O_KI + SZ_T;       // V, then (own rows) dY_v
constexpr int O_DO = O_V + SZ_T;
constexpr int O_NW = O_DO + SZ_T;      // -W
constexpr int O_NU = O_NW + SZ_T;      // -U
constexpr int O_E = O_NU + SZ_T;
constexpr int O_NDE = O_E + SZ_T;      // -dE, then dY_k
constexpr int O_R = O_NDE + SZ_T;      // [value][channel]: S_m, then dS_m
constexpr int O_A = O_R + DD * LR * 2; // fp32 A (strict lower)
constexpr int O_T = O_A + SZ_F;        // fp32 T
constexpr int O_AQ = O_T + SZ_F;       // Aqk^T  [j][i]
constexpr int O_TT = O_AQ + SZ_S;      // T^T    [j][i]
constexpr int O_TB = O_TT + SZ_S;      // (T Diag(beta))^T
constexpr int O_DAQ = O_TB + SZ_S;     // dAqk^T
constexpr int O_DA = O_DAQ + SZ_S;     // dA^T
constexpr int O_BETA = O_DA + SZ_S;    // f32[32]
constexpr int O_ER = O_BETA + 128;     // f32[128] e^r
constexpr int O_DL = O_ER + 512;       // f32[128] e^{b_L - r}
constexpr int O_RP = O_DL + 512;       // f32[8][128] per-wave partials of sum_v dS_m S_m
constexpr int NDBP = 19;               // dbeta partial slots: 8 (dY_v), 8 (dY_k), 3 (dL)
constexpr int O_DBP = O_RP + 4096;     // f32[19][32]
constexpr int O_GP = O_DBP + NDBP * 128;   // f32[8][32] per-token dlog alpha partials (per-head gate)
constexpr int O_FLAG = O_GP + 1024;
constexpr int LDS_BYTES = O_FLAG + 16;
static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
static_assert((KDA_LPT_MAX + 1) * 4 <= SZ_T, "length ranking in the E buffer");

// One chunk's operand buffers.  The reverse sweep uses set 0; the forward
// sweep alternates set 0 with buffers it has no other use for, so that the
// next chunk's operands and T are formed while this chunk's state update runs.
struct Set {
  int kg, ki, v, beta, er, dl, tt;   // tb = tt + SZ_S
};
constexpr Set SET0{O_KG, O_KI, O_V, O_BETA, O_ER, O_DL, O_TT};
constexpr Set SET1{O_QG, O_DO, O_NU, O_DBP, O_DBP + 128, O_DBP + 640, O_DAQ};
static_assert(O_TB == O_TT + SZ_S && O_DA == O_DAQ + SZ_S, "T buffer pairs");
// Shared staging of a chunk's loaded inputs (E, -dE and R are free from the
// time a chunk's inputs are staged until they are unpacked): q, k, v and dO as
// bf16 [token][LS], then the gates as fp32 [token][LG] (a per-head gate:
// f32[32]).  With 288-byte rows the four rows of a transpose read fall in
// distinct banks.
constexpr int LS = DD + 16;
constexpr int LG = DD + 4;
constexpr int STG_T = BC * LS * 2;
constexpr int O_SG = O_E + 4 * STG_T;
static_assert(O_NDE == O_E + SZ_T && O_R == O_NDE + SZ_T &&
              O_SG + BC * LG * 4 <= O_R + DD * LR * 2, "input staging");
static_assert(640 + 512 <= NDBP * 128, "second set's small buffers");

typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef LDS uint16_t* lb;
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ i16x4 tr(const LDS uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(p));
}
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b) {
  u32x4 w{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
          pack_bf16x2(b[2], b[3])};
  return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ f32x4 unpack4(u32x2 w) {
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
               __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
}

// Lane coordinates: n = lane % 16, g = lane / 16, wave w.
struct Ln {
  int n, g, w, l;
};

// The lane coordinates, re-materialised after every barrier: the volatile asm
// keeps the compiler from hoisting lane-dependent LDS addresses out of the
// chunk loops, where they would hold registers for the whole kernel.
__device__ __forceinline__ Ln fresh() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return Ln{l & 15, l >> 4, __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), l};
}

// Operand reads.  Natural k order: lane (n, g) holds k0 + 8g + e, e < 8.
// X[row0 + n][k0 + 8g + e]
__device__ __forceinline__ bf16x8 rd_row(const LDS uint16_t* X, int ld, int row0, int k0,
                                         const Ln& L) {
  return *(const LDS bf16x8*)(X + (row0 + L.n) * ld + k0 + 8 * L.g);
}
// X[k0 + 8g + e][col0 + n]
__device__ __forceinline__ bf16x8 rd_tr(const LDS uint16_t* X, int ld, int k0, int col0,
                                        const Ln& L) {
  const LDS uint16_t* p = X + (k0 + 8 * L.g + (L.n >> 2)) * ld + col0 + 4 * (L.n & 3);
  return cat(tr(p), tr(p + 4 * ld));
}
// Relabelled k order, to pair with two stacked accumulator tiles in registers:
// position 8g + e holds k0 + 4g + e (e < 4) and k0 + 16 + 4g + e - 4 (e >= 4).
__device__ __forceinline__ bf16x8 rd_rowp(const LDS uint16_t* X, int ld, int row0, int k0,
                                          const Ln& L) {
  const LDS uint16_t* p = X + (row0 + L.n) * ld + k0 + 4 * L.g;
  return cat(*(const LDS i16x4*)p, *(const LDS i16x4*)(p + 16));
}
__device__ __forceinline__ bf16x8 rd_trp(const LDS uint16_t* X, int ld, int k0, int col0,
                                         const Ln& L) {
  const LDS uint16_t* p = X + (k0 + 4 * L.g + (L.n >> 2)) * ld + col0 + 4 * (L.n & 3);
  return cat(tr(p), tr(p + 16 * ld));
}
// Accumulator tile (rows row0 + 4g + r, column col0 + n) stored transposed:
// Xt[col0 + n][row0 + 4g + r], one 8-byte write.
__device__ __forceinline__ void st_t(LDS uint16_t* Xt, int ld, int col0, int row0, f32x4 v,
                                     const Ln& L) {
  *(LDS u32x2*)(Xt + (col0 + L.n) * ld + row0 + 4 * L.g) =
      u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}
__device__ __forceinline__ void st_raw(LDS uint16_t* Xt, int ld, int col0, int row0, u32x2 v,
                                       const Ln& L) {
  *(LDS u32x2*)(Xt + (col0 + L.n) * ld + row0 + 4 * L.g) = v;
}
__device__ __forceinline__ u32x2 ld_raw(const LDS uint16_t* Xt, int ld, int col0, int row0,
                                        const Ln& L) {
  return *(const LDS u32x2*)(Xt + (col0 + L.n) * ld + row0 + 4 * L.g);
}

// One reduce-scatter step inside 16-lane rows: lanes with `hi` keep b, the
// others a, each adding the partner's copy (DPP pattern CTRL pairs every lane
// with one of the other kind).
template <int CTRL>
__device__ __forceinline__ float rs_step(float a, float b, bool hi) {
  const float keep = hi ? b : a, send = hi ? a : b;
  return keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xf, 0xf, false));
}

// Sums over the 16 lanes of each DPP row of the 32 values x[cb][r] (rows
// 16cb + 4g + r of a column-per-lane layout), scattered: lane n ends with the
// sums of rows 16cb + 4g + 2(n % 2) + {0, 1}, cb = 4[n >= 8] + 2[n % 8 >= 4] +
// [n % 4 >= 2].  Four butterfly steps (mirror, half mirror, quad reversal,
// pair swap), 30 DPP adds in all instead of 128.
__device__ __forceinline__ f32x2 row_sums_scatter(const f32x4 x[8], int n) {
  float a[16], b[8], c[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 4; ++r) a[4 * k + r] = rs_step<0x140>(x[k][r], x[k + 4][r], n >= 8);
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int r = 0; r < 4; ++r) b[4 * k + r] = rs_step<0x141>(a[4 * k + r], a[4 * (k + 2) + r], (n & 7) >= 4);
#pragma unroll
  for (int r = 0; r < 4; ++r) c[r] = rs_step<0x1B>(b[r], b[4 + r], (n & 3) >= 2);
  return f32x2{rs_step<0xB1>(c[0], c[2], n & 1), rs_step<0xB1>(c[1], c[3], n & 1)};
}

// One chunk's inputs as loaded: each wave loads its own 32-token slice of its
// 16 channels (value columns), 16 bytes per lane and tensor: bf16 tensors as
// token L / 2, columns 8 (L % 2) .. +7; the gates as tokens L / 4 and 16 + L / 4,
// columns 4 (L % 4) .. +3 (per-head gates: token L, L < 32).  Nothing touches
// these registers until the chunk is unpacked, so the prefetch is never
// waited for where it is issued.
struct In {
  u32x4 q, k, v, o;
  f32x4 g0, g1;
};
// The lane's elements in the accumulator layout: tokens 16I + 4g + r of
// column 16w + n, bf16 as two packed dwords per I.
struct Ch {
  u32x2 q[2], k[2], v[2], o[2];
  float gt[2][4];
};

// Buffer views: a workgroup-uniform base and byte limit, a 32-bit lane offset
// and a uniform offset per access; reads at or past the limit return zero and
// writes there are dropped.  A chunk's view of a [rows, H, width] tensor starts
// at its first row of head h and ends after its last valid row, so the
// padding rows of a partial chunk need no test.
constexpr int BUF_FLAGS = 0x00020000;
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc chunk_view(const void* p, size_t tok0, int L, int H, int h,
                                           int width, int esz) {
  const char* base = (const char*)p + (tok0 * H + h) * (size_t)width * esz;
  const int bytes = L > 0 ? (int)(((size_t)(L - 1) * H * width + width) * esz) : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, BUF_FLAGS);
}
__device__ __forceinline__ void st_f32(Rsrc r, uint32_t off, uint32_t soff, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, soff, 0);
}

// A chunk's inputs, whole rows at a time: wave w loads tokens 4w .. 4w+3,
// lane l 16 bytes of token 4w + l/16 (the fp32 gates in two loads, the row's
// first and second halves), so that a load covers four whole rows.  A
// per-head gate is loaded by wave 0 alone.
template <bool SG>
__device__ __forceinline__ void load_in(In& x, const uint16_t* q, const uint16_t* k,
                                        const uint16_t* v, const uint16_t* dout, const float* g,
                                        size_t tok0, int L, int H, int h, bool rev, const Ln& ln) {
  const Rsrc rq = chunk_view(q, tok0, L, H, h, DD, 2), rk = chunk_view(k, tok0, L, H, h, DD, 2);
  const Rsrc rv = chunk_view(v, tok0, L, H, h, DD, 2), ro = chunk_view(dout, tok0, L, H, h, DD, 2);
  const Rsrc rg = chunk_view(g, tok0, L, H, h, SG ? 1 : DD, 4);
  const uint32_t row = 4 * ln.w + (ln.l >> 4), c = ln.l & 15;
  const uint32_t ob = 2 * (row * H * DD + 8 * c);
  const u32x4 z{0u, 0u, 0u, 0u};
  x.q = rev ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, ob, 0, 0)) : z;
  x.k = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, ob, 0, 0));
  x.v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, ob, 0, 0));
  x.o = rev ? __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, ob, 0, 0)) : z;
  x.g0 = f32x4{0.f, 0.f, 0.f, 0.f};
  x.g1 = f32x4{0.f, 0.f, 0.f, 0.f};
  if (SG) {
    if (ln.w == 0)
      x.g0[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, 4 * (uint32_t)(ln.l * H), 0, 0));
  } else {
    const uint32_t og = 4 * (row * H * DD + 4 * c);
    x.g0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, og, 0, 0));
    x.g1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, og, 256, 0));
  }
}

// The loaded rows into the shared staging.  A barrier must separate this from
// the unpacking reads, and those from the next staging.
template <bool SG>
__device__ __forceinline__ void stage(LDS char* lds, const In& x, bool rev, const Ln& ln) {
  const int row = 4 * ln.w + (ln.l >> 4), c = ln.l & 15;
  LDS char* s = lds + O_E + (row * LS + 8 * c) * 2;
  if (rev) *(LDS u32x4*)(s) = x.q;
  *(LDS u32x4*)(s + STG_T) = x.k;
  *(LDS u32x4*)(s + 2 * STG_T) = x.v;
  if (rev) *(LDS u32x4*)(s + 3 * STG_T) = x.o;
  LDS float* sg = (LDS float*)(lds + O_SG);
  if (SG) {
    if (ln.w == 0 && ln.l < BC) sg[ln.l] = x.g0[0];
  } else {
    *(LDS f32x4*)(sg + row * LG + 4 * c) = x.g0;
    *(LDS f32x4*)(sg + row * LG + 64 + 4 * c) = x.g1;
  }
}

// The wave's columns of the staged chunk in the accumulator layout: the
// transpose read gives lane n of group g tokens 4g .. 4g+3 of column 16w + n.
template <bool SG>
__device__ __forceinline__ Ch unstage(const LDS char* lds, bool rev, const Ln& ln) {
  const LDS float* sg = (const LDS float*)(lds + O_SG);
  Ch c;
#pragma unroll
  for (int I = 0; I < 2; ++I) {
    const int e = (16 * I + 4 * ln.g + (ln.n >> 2)) * LS + 16 * ln.w + 4 * (ln.n & 3);
    auto rd = [&](int t) {
      return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                           (LDS i16x4*)((const LDS uint16_t*)(lds + O_E + t * STG_T) + e)));
    };
    c.k[I] = rd(1);
    c.v[I] = rd(2);
    c.q[I] = rev ? rd(0) : u32x2{0u, 0u};
    c.o[I] = rev ? rd(3) : u32x2{0u, 0u};
#pragma unroll
    for (int r = 0; r < 4; ++r)
      c.gt[I][r] = SG ? sg[16 * I + 4 * ln.g + r] : sg[(16 * I + 4 * ln.g + r) * LG + 16 * ln.w + ln.n];
  }
  return c;
}

// The value held by lane group g ^ 1 (g ^ 2) in the lane's column.  gfx950's
// permlane16 (permlane32) swap, given one register as both operands, returns
// it with rows 1 and 3 (lanes 32..63) taken from rows 0 and 2 (lanes 0..31)
// as its first result and the converse as its second.
__device__ __forceinline__ float from_g1(float x, const Ln& ln) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float((ln.g & 1) ? r[0] : r[1]);
}
__device__ __forceinline__ float from_g2(float x, const Ln& ln) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((ln.g & 2) ? r[0] : r[1]);
}

// b - r for the lane's eight elements and whether any lies beyond RANGE, with
// r = b_15; also e^r and e^{b_L - r} of the lane's channel.  The in-chunk
// prefix sums: running sums over the lane's four tokens, then over the four
// lane groups by two swaps (a pair's sum, then the other pair's).
__device__ __forceinline__ bool prefix(const Ch& x, f32x4 bm[2], float& er, float& dl,
                                       const Ln& ln) {
  f32x4 p[2];
  float ex[2], all[2];
#pragma unroll
  for (int I = 0; I < 2; ++I) {
    p[I][0] = x.gt[I][0];
#pragma unroll
    for (int s = 1; s < 4; ++s) p[I][s] = p[I][s - 1] + x.gt[I][s];
    const float t = p[I][3];
    const float o1 = from_g1(t, ln);
    const float pair = t + o1;                  // groups 2h and 2h + 1
    const float lo = (ln.g & 1) ? o1 : 0.f;     // group g - 1 of the pair
    const float o2 = from_g2(pair, ln);
    ex[I] = (ln.g & 2) ? o2 + lo : lo;          // groups before g
    all[I] = pair + o2;                         // all sixteen tokens
  }
  const float r = all[0];                       // b_15
  const float bl = all[0] + all[1];             // b_31
  bool bad = false;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bm[0][e] = (p[0][e] + ex[0]) - r;
    bm[1][e] = ((p[1][e] + ex[1]) + all[0]) - r;
    bad |= !(fabsf(bm[0][e]) <= RANGE) || !(fabsf(bm[1][e]) <= RANGE);
  }
  er = __expf(r);
  dl = __expf(bl - r);
  return bad;
}

// Lower-triangle 16x16 tiles of a 32x32 matrix: (0,0), (1,0), (1,1).
__device__ __forceinline__ int tile_I(int t) { return t == 0 ? 0 : 1; }
__device__ __forceinline__ int tile_J(int t) { return t == 2 ? 1 : 0; }

// The WY inverse of one chunk on one wave, fp32: N = Diag(beta) A with
// A = strict_tril(KG KI^T), T = (I + N)^{-1}.
//  * The three lower 16x16 tiles of A share their operand reads; N^T goes to
//    LDS ([j][i], fp32).
//  * Diagonal blocks by forward substitution: lanes with g even take column n
//    of T_00, lanes with g odd column n of T_11, the whole column in
//    registers, every later row updated as soon as a row is final.  The rows
//    of N^T are read three rows ahead of their use (the scheduling fences keep
//    the compiler from sinking the reads back), so the LDS latency stays off
//    the substitution's chain.
//  * X = N_10 T_00 and T_10 = -T_11 X as fp32 MFMAs (16x16x4, k step r takes
//    matrix index 4g + r): every operand is one LDS read or the lane's own
//    accumulator register.
// Writes T^T and (T Diag(beta))^T as bf16 into the set's buffers.  The tiles
// and the rest are separate calls, so that the forward sweep can give the
// tiles to another wave.
__device__ __forceinline__ void tiles_nt(LDS char* lds, Set st, const Ln& ln) {
  LDS float* Nt = (LDS float*)(lds + O_A);
  const LDS float* beta = (const LDS float*)(lds + st.beta);
  {
    f32x4 a[3] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                  f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x8 g0 = rd_tr((lb)(lds + st.kg), LT, 32 * kc, 0, ln);
      const bf16x8 g1 = rd_tr((lb)(lds + st.kg), LT, 32 * kc, 16, ln);
      const bf16x8 i0 = rd_tr((lb)(lds + st.ki), LT, 32 * kc, 0, ln);
      const bf16x8 i1 = rd_tr((lb)(lds + st.ki), LT, 32 * kc, 16, ln);
      a[0] = mma(g0, i0, a[0]);
      a[1] = mma(g1, i0, a[1]);
      a[2] = mma(g1, i1, a[2]);
    }
#pragma unroll
    for (int t = 0; t < 3; ++t) {
      const int I = tile_I(t), J = tile_J(t);
      f32x4 acc = a[t];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (I > J || 4 * ln.g + r > ln.n) ? acc[r] : 0.f;
      const f32x4 bt = *(const LDS f32x4*)(beta + 16 * I + 4 * ln.g);
      *(LDS f32x4*)(Nt + (16 * J + ln.n) * LA + 16 * I + 4 * ln.g) = acc * bt;
    }
  }
}
__device__ __forceinline__ void invert_nt(LDS char* lds, Set st, const Ln& ln) {
  const LDS float* Nt = (const LDS float*)(lds + O_A);
  LDS float* Tf = (LDS float*)(lds + O_T);
  const LDS float* beta = (const LDS float*)(lds + st.beta);
  const int b = ln.g & 1, off = 16 * b, j = ln.n;
  const LDS float* Nb = Nt + off * LA + off;   // row m: column m of N_bb
  f32x4 R[15][4];
  auto ldrow = [&](int m) {
#pragma unroll
    for (int q = (m + 1) >> 2; q < 4; ++q) R[m][q] = *(const LDS f32x4*)(Nb + m * LA + 4 * q);
  };
  float x[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
  ldrow(0);
  ldrow(1);
  ldrow(2);
#pragma unroll
  for (int m = 0; m < 15; ++m) {
    if (m + 3 < 15) ldrow(m + 3);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = m + 1; i < 16; ++i) x[i] -= R[m][i >> 2][i & 3] * x[m];
  }
  __builtin_amdgcn_sched_barrier(0);
  if (ln.g < 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) Tf[(off + i) * LA + off + j] = x[i];
    const float bj = beta[off + j];
    LDS uint16_t* tt = (lb)(lds + st.tt) + (off + j) * LT + off;
    LDS uint16_t* tb = (lb)(lds + st.tt + SZ_S) + (off + j) * LT + off;
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      *(LDS u32x2*)(tt + e) = u32x2{pack_bf16x2(x[e], x[e + 1]), pack_bf16x2(x[e + 2], x[e + 3])};
      *(LDS u32x2*)(tb + e) = u32x2{pack_bf16x2(bj * x[e], bj * x[e + 1]),
                                    pack_bf16x2(bj * x[e + 2], bj * x[e + 3])};
    }
  }
  f32x4 X{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r)
    X = mma4(Nt[(4 * ln.g + r) * LA + 16 + ln.n], Tf[(4 * ln.g + r) * LA + ln.n], X);
  const f32x4 t11 = *(const LDS f32x4*)(Tf + (16 + ln.n) * LA + 16 + 4 * ln.g);
  f32x4 t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 4; ++r) t = mma4(-t11[r], X[r], t);
  st_t((lb)(lds + st.tt), LT, 0, 16, t, ln);
  st_t((lb)(lds + st.tt + SZ_S), LT, 0, 16, t * beta[j], ln);
}

// Stores a wave's 32 x 16 fp32 tile (accumulator layout: tokens 16I + 4g + r,
// column 16w + n) to a chunk view of a [rows, H, 128] tensor: eight 4-byte
// stores per lane, each instruction writing the wave's 64 bytes of four token
// rows; the view drops the padding rows.  (Staging the tile through LDS into
// 16-byte stores of the same rows measured slower: its LDS round trip sat in
// the epilogue.)
__device__ __forceinline__ void store_tile(Rsrc rv, const f32x4 x[2], int H, const Ln& ln) {
#pragma unroll
  for (int I = 0; I < 2; ++I)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      st_f32(rv, 4 * (uint32_t)((16 * I + 4 * ln.g + r) * H * DD + 16 * ln.w + ln.n), 0, x[I][r]);
}

// Writes every input prep product of one chunk: KG, KI, V (and, reverse sweep,
// QG and dO) as [channel][token] bf16, e^r and e^{b_L - r} of the lane's channel.
__device__ __forceinline__ void prep_store(LDS char* lds, Set st, const Ch& x,
                                           const f32x4 bm[2], float er, float dl, float scale,
                                           bool rev, const Ln& ln) {
#pragma unroll
  for (int I = 0; I < 2; ++I) {
    const f32x4 kf = unpack4(x.k[I]);
    f32x4 p, pi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = __expf(bm[I][e]);
      pi[e] = __expf(-bm[I][e]);
    }
    st_t((lb)(lds + st.kg), LT, 16 * ln.w, 16 * I, kf * p, ln);
    st_t((lb)(lds + st.ki), LT, 16 * ln.w, 16 * I, kf * pi, ln);
    st_raw((lb)(lds + st.v), LT, 16 * ln.w, 16 * I, x.v[I], ln);
    if (rev) {
      st_t((lb)(lds + O_QG), LT, 16 * ln.w, 16 * I, unpack4(x.q[I]) * p * scale, ln);
      st_raw((lb)(lds + O_DO), LT, 16 * ln.w, 16 * I, x.o[I], ln);
    }
  }
  if (ln.g == 0) {
    ((LDS float*)(lds + st.er))[16 * ln.w + ln.n] = er;
    ((LDS float*)(lds + st.dl))[16 * ln.w + ln.n] = dl;
  }
}

// Tile t (0..2) of A = strict_tril(KG KI^T) or, qk, of Aqk = tril(QG KI^T)
// (bf16, transposed).  A is stored fp32, row-major, for dbeta.
__device__ __forceinline__ void tile_a(LDS char* lds, Set st, bool qk, int t, const Ln& ln) {
  const int I = tile_I(t), J = tile_J(t);
  const lb X = (lb)(lds + (qk ? O_QG : st.kg));
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
    acc = mma(rd_tr(X, LT, 32 * kc, 16 * I, ln), rd_tr((lb)(lds + st.ki), LT, 32 * kc, 16 * J, ln),
              acc);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * I + 4 * ln.g + r, j = 16 * J + ln.n;
    acc[r] = (qk ? i >= j : i > j) ? acc[r] : 0.f;
  }
  if (qk) {
    st_t((lb)(lds + O_AQ), LT, 16 * J, 16 * I, acc, ln);
  } else {
    LDS float* A = (LDS float*)(lds + O_A);
#pragma unroll
    for (int r = 0; r < 4; ++r) A[(16 * I + 4 * ln.g + r) * LA + 16 * J + ln.n] = acc[r];
  }
}

// Copies T^T and (T Diag(beta))^T between LDS and a workspace slot: thread
// t moves four elements of row (t / 8) % 32 of buffer t / 256.
__device__ __forceinline__ LDS u32x2* t_part(LDS char* lds, Set st) {
  const int t = threadIdx.x;
  return (LDS u32x2*)((lb)(lds + st.tt + (t >> 8) * SZ_S) + ((t >> 3) & 31) * LT + 4 * (t & 7));
}

// U = T Diag(beta) V (own value columns, registers; -U also to LDS) and
// W = T Diag(beta) KG (own key channels; -W to LDS).
__device__ __forceinline__ void tiles_uw(LDS char* lds, Set st, f32x4 U[2], bool store_u,
                                         const Ln& ln) {
#pragma unroll
  for (int I = 0; I < 2; ++I) {
    const bf16x8 tb = rd_tr((lb)(lds + st.tt + SZ_S), LT, 0, 16 * I, ln);
    U[I] = mma(tb, rd_row((lb)(lds + st.v), LT, 16 * ln.w, 0, ln), f32x4{0.f, 0.f, 0.f, 0.f});
    const f32x4 W = mma(tb, rd_row((lb)(lds + st.kg), LT, 16 * ln.w, 0, ln),
                        f32x4{0.f, 0.f, 0.f, 0.f});
    st_t((lb)(lds + O_NW), LT, 16 * ln.w, 16 * I, -W, ln);
    if (store_u) st_t((lb)(lds + O_NU), LT, 16 * ln.w, 16 * I, -U[I], ln);
  }
}

// y_t = sum_{i >= t} x_i + sum_{i < t} z_i over the chunk's tokens
// (accumulator layout): running sums over the lane's four tokens (x from the
// last, z exclusive from the first), joined across the four lane groups by two
// swaps and across the chunk's halves by the half totals.
__device__ __forceinline__ void suffix_prefix(const f32x4 x[2], const f32x4 z[2], f32x4 y[2],
                                              const Ln& ln) {
  f32x4 sx[2], pz[2];
  float xa[2], zb[2], xall[2], zall[2];
#pragma unroll
  for (int I = 0; I < 2; ++I) {
    sx[I][3] = x[I][3];
#pragma unroll
    for (int s = 2; s >= 0; --s) sx[I][s] = sx[I][s + 1] + x[I][s];
    pz[I][0] = 0.f;
#pragma unroll
    for (int s = 1; s < 4; ++s) pz[I][s] = pz[I][s - 1] + z[I][s - 1];
    const float tx = sx[I][0], tz = pz[I][3] + z[I][3];
    const float ox = from_g1(tx, ln), oz = from_g1(tz, ln);
    const float px = tx + ox, qz = tz + oz;          // pair sums
    const float hx = (ln.g & 1) ? 0.f : ox;          // group g + 1 of the pair
    const float lz = (ln.g & 1) ? oz : 0.f;          // group g - 1 of the pair
    const float o2x = from_g2(px, ln), o2z = from_g2(qz, ln);
    xa[I] = (ln.g & 2) ? hx : o2x + hx;              // x over the groups after g
    zb[I] = (ln.g & 2) ? o2z + lz : lz;              // z over the groups before g
    xall[I] = px + o2x;
    zall[I] = qz + o2z;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    y[0][s] = ((sx[0][s] + xa[0]) + xall[1]) + (pz[0][s] + zb[0]);
    y[1][s] = (sx[1][s] + xa[1]) + ((pz[1][s] + zb[1]) + zall[0]);
  }
}

template <bool SG>
__global__ __launch_bounds__(NT, 1) void bwd_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    const float* __restrict__ S0, const uint16_t* __restrict__ dout,
    const float* __restrict__ dSf, float* __restrict__ dq, float* __restrict__ dk,
    float* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta,
    float* __restrict__ dS0, const int32_t* __restrict__ cu, int T, int H, float scale,
    uint32_t* __restrict__ states, int* __restrict__ flags, int spin) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  LDS char* lds = (LDS char*)lds_raw;
  Ln ln = fresh();
  const int h = blockIdx.x % H;
  int sq = blockIdx.x / H;
  // Packed sequences: workgroup b takes head b % H of the (b / H)-th longest
  // sequence (ties by index; ranked in LDS, up to KDA_LPT_MAX sequences), so
  // that long chains start first.
  if (cu && (int)(gridDim.x / H) <= KDA_LPT_MAX) {
    const int N = gridDim.x / H;
    LDS int* lens = (LDS int*)(lds + O_E);
    LDS int* pick = lens + KDA_LPT_MAX;
    for (int m = threadIdx.x; m < N; m += NT) lens[m] = cu[m + 1] - cu[m];
    __syncthreads();
    for (int m = threadIdx.x; m < N; m += NT) {
      const int lm = lens[m];
      int rank = 0;
      for (int j = 0; j < N; ++j) rank += (lens[j] > lm) || (lens[j] == lm && j < m);
      if (rank == sq) *pick = m;
    }
    __syncthreads();
    sq = *pick;
    __syncthreads();   // the LDS is the kernel's from here on
  }
  const int nh = sq * H + h;
  size_t t0;
  int len;
  if (cu) {
    t0 = (size_t)cu[sq];
    len = cu[sq + 1] - cu[sq];
  } else {
    t0 = (size_t)sq * T;
    len = T;
  }
  const int nc = (len + BC - 1) / BC;
  // chunk m's workspace slot: S_c in the lanes' own order, then T^T and (T Diag(beta))^T
  uint32_t* slot0 = states + ((size_t)sq + t0 / BC) * H * SLOT_DW + (size_t)h * SLOT_DW;
  auto slot = [&](int m, int cb, const Ln& L) {
    return (u32x2*)(slot0 + (size_t)m * H * SLOT_DW) + (L.w * 8 + cb) * 64 + L.l;
  };
  auto tslot = [&](int m) {
    return (u32x2*)(slot0 + (size_t)m * H * SLOT_DW + ST_DW) + threadIdx.x;
  };
  LDS float* ER = (LDS float*)(lds + O_ER);
  LDS float* DL = (LDS float*)(lds + O_DL);
  LDS float* BETA = (LDS float*)(lds + O_BETA);
  LDS float* DBP = (LDS float*)(lds + O_DBP);
  LDS float* RP = (LDS float*)(lds + O_RP);
  LDS float* GP = (LDS float*)(lds + O_GP);
  LDS int* FLAG = (LDS int*)(lds + O_FLAG);
  LDS int* TFLAG = FLAG + 1;   // forward sweep: index of the chunk whose A tiles are in O_A
  // upper blocks of the [j][i] 32x32 buffers stay zero
  for (int e = threadIdx.x; e < 5 * 256; e += NT) {
    const int b = e >> 8, j = 16 + ((e >> 4) & 15), i = e & 15;
    ((lb)(lds + O_AQ + b * SZ_S))[j * LT + i] = 0;
  }
  if (threadIdx.x == 0) {
    *FLAG = 0;
    *TFLAG = -1;
  }
  const int col = 16 * ln.w + ln.n;   // the lane's value column / key channel
  const size_t sbase = (size_t)nh * DD * DD;

  // ------------------------------------------------------------ forward sweep
  f32x4 S[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[cb][r] = S0 ? S0[sbase + (size_t)(16 * cb + 4 * ln.g + r) * DD + col] : 0.f;
  __syncthreads();
  ln = fresh();
  // the next chunk's inputs (and, reverse sweep, its stored state and T) load
  // while this one is computed
  auto clen = [&](int mm) { return len - BC * mm < BC ? len - BC * mm : BC; };
  In xn;
  float bn = 0.f;
  auto fetch = [&](int mm, bool rev, const Ln& ll) {
    const int L = clen(mm);
    const size_t tok0 = t0 + (size_t)BC * mm;
    load_in<SG>(xn, q, k, v, dout, g, tok0, L, H, h, rev, ll);
    bn = (ll.w == 0 && ll.l < L) ? beta[(tok0 + ll.l) * H + h] : 0.f;
  };
  if (nc > 0) fetch(0, false, ln);
  // chunk mm's operands into set st from the prefetched inputs, then the next fetch
  auto prep1 = [&](int mm, Set st, const Ln& ll) {
    const Ch x = unstage<SG>(lds, false, ll);
    if (ll.w == 0 && ll.l < BC) ((LDS float*)(lds + st.beta))[ll.l] = bn;
    if (mm + 1 < nc) fetch(mm + 1, false, ll);
    f32x4 bm[2];
    float er, dl;
    if (prefix(x, bm, er, dl, ll)) *FLAG = 1;
    prep_store(lds, st, x, bm, er, dl, scale, false, ll);
  };
  // T of the chunk whose operands are in set st, on the last wave
  auto solve1 = [&](Set st, const Ln& ll) {
    tiles_nt(lds, st, ll);
    invert_nt(lds, st, ll);
  };
  if (nc > 0) {
    stage<SG>(lds, xn, false, ln);
    __syncthreads();
    ln = fresh();
    prep1(0, SET0, ln);
    __syncthreads();
    ln = fresh();
    if (ln.w == NW - 1 && !*FLAG) solve1(SET0, ln);
    if (nc > 1) stage<SG>(lds, xn, false, ln);
    __syncthreads();
    ln = fresh();
  }
  for (int m = 0; m < nc; ++m) {
    const Set cur = (m & 1) ? SET1 : SET0, nxt = (m & 1) ? SET0 : SET1;
    if (*FLAG) break;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      *slot(m, cb, ln) = u32x2{pack_bf16x2(S[cb][0], S[cb][1]), pack_bf16x2(S[cb][2], S[cb][3])};
    *tslot(m) = *t_part(lds, cur);
    f32x4 Sm[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      Sm[cb] = S[cb] * *(const LDS f32x4*)((const LDS float*)(lds + cur.er) + 16 * cb + 4 * ln.g);
    f32x4 U[2];
    tiles_uw(lds, cur, U, false, ln);
    if (m + 1 < nc) prep1(m + 1, nxt, ln);
    __syncthreads();   // #a: -W; the next chunk's operands
    ln = fresh();
    // the next chunk's A tiles on the second-to-last wave before its state update,
    // published to the last wave, which inverts after its own update
    const bool solve = m + 1 < nc && !*FLAG;
    if (ln.w == NW - 2 && solve) {
      tiles_nt(lds, nxt, ln);
      __hip_atomic_store(TFLAG, m + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    // E = U - W S_m (own value columns); S_{c+1} = Diag(e^{b_L - r}) (S_m + KI^T E)
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x8 sb = pack8(Sm[2 * kc], Sm[2 * kc + 1]);
#pragma unroll
      for (int I = 0; I < 2; ++I) U[I] = mma(rd_trp((lb)(lds + O_NW), LT, 32 * kc, 16 * I, ln), sb, U[I]);
    }
    const bf16x8 eb = pack8(U[0], U[1]);
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
      S[cb] = mma(rd_rowp((lb)(lds + cur.ki), LT, 16 * cb, 0, ln), eb, Sm[cb]) *
              *(const LDS f32x4*)((const LDS float*)(lds + cur.dl) + 16 * cb + 4 * ln.g);
    if (ln.w == NW - 1 && solve) {
      // a wait of at most `spin` polls; past it the wave forms the tiles itself
      // (the same values, so a late second write changes nothing)
      bool got = false;
      for (int it = 0; it < spin; ++it) {
        got = __hip_atomic_load(TFLAG, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == m + 1;
        if (got) break;
        __builtin_amdgcn_s_sleep(1);
      }
      if (!got) tiles_nt(lds, nxt, ln);
      invert_nt(lds, nxt, ln);
    }
    if (m + 2 < nc) stage<SG>(lds, xn, false, ln);
    __syncthreads();   // #b: the next chunk's T and staged inputs; this chunk's buffers are free
    ln = fresh();
  }
  if (*FLAG) {
    if (threadIdx.x == 0) flags[nh] = 1;
    return;
  }
  if (threadIdx.x == 0) flags[nh] = 0;

  // ------------------------------------------------------------ reverse sweep
  f32x4 dS[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dS[cb][r] = dSf ? dSf[sbase + (size_t)(16 * cb + 4 * ln.g + r) * DD + col] : 0.f;
  // dbeta (and a per-head gate's dlog alpha) of chunk mm from the partials
  auto finish_rows = [&](int mm, const Ln& ll) {
    if (ll.w == NW - 1 && ll.l < BC) {
      const int L = clen(mm);
      if (ll.l < L) {
        const size_t row = (t0 + (size_t)BC * mm + ll.l) * H + h;
        float s = 0.f;
        for (int p = 0; p < NDBP; ++p) s += DBP[p * BC + ll.l];
        dbeta[row] = s;
        if (SG) {
          float t = 0.f;
          for (int p = 0; p < NW; ++p) t += GP[p * BC + ll.l];
          dg[row] = t;
        }
      }
    }
  };
  u32x2 Scn[8], Tn;
  // the next chunk's state and T, in two batches (the inputs come first)
  auto fetch_s = [&](int mm, int c0, const Ln& L) {
#pragma unroll
    for (int cb = c0; cb < c0 + 4; ++cb) Scn[cb] = *slot(mm, cb, L);
    if (c0) Tn = *tslot(mm);
  };
  if (nc > 0) {
    fetch(nc - 1, true, ln);
    fetch_s(nc - 1, 0, ln);
    fetch_s(nc - 1, 4, ln);
    stage<SG>(lds, xn, true, ln);
    __syncthreads();
    ln = fresh();
  }
  for (int m = nc - 1; m >= 0; --m) {
    const int L = clen(m);
    const size_t tok0 = t0 + (size_t)BC * m;
    const Ch x = unstage<SG>(lds, true, ln);
    const u32x2 o0 = x.o[0], o1 = x.o[1];
    if (ln.w == 0 && ln.l < BC) BETA[ln.l] = bn;
    u32x2 Sc[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) Sc[cb] = Scn[cb];
    *t_part(lds, SET0) = Tn;
    f32x4 bm[2];
    float er, dl;
    prefix(x, bm, er, dl, ln);
    prep_store(lds, SET0, x, bm, er, dl, scale, true, ln);
    __syncthreads();   // #1: the chunk's operands, T
    ln = fresh();
    if (m + 1 < nc) finish_rows(m + 1, ln);
    // dS_m = Diag(e^{b_L - r}) dS;  S_m = Diag(e^r) S_c to R ([value][channel]);
    // sum_v dS_m S_m over the lane's columns into the partials (the decay of
    // the incoming state over the chunk, part of every token's dlog alpha)
    {
      // every factor is read before the first store (the compiler cannot
      // tell the stores from the reads and would otherwise wait on each)
      f32x4 pr[8], dlf[8], erf[8];
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        dlf[cb] = *(const LDS f32x4*)(DL + 16 * cb + 4 * ln.g);
        erf[cb] = *(const LDS f32x4*)(ER + 16 * cb + 4 * ln.g);
      }
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        dS[cb] *= dlf[cb];
        const f32x4 sm = unpack4(Sc[cb]) * erf[cb];
        st_t((lb)(lds + O_R), LR, 16 * ln.w, 16 * cb, sm, ln);
        pr[cb] = dS[cb] * sm;
      }
      const f32x2 rs = row_sums_scatter(pr, ln.n);
      const int cb = 4 * (ln.n >= 8) + 2 * ((ln.n & 7) >= 4) + ((ln.n & 3) >= 2);
      *(LDS f32x2*)(RP + ln.w * DD + 16 * cb + 4 * ln.g + 2 * (ln.n & 1)) = rs;
    }
    if (ln.w < 6) tile_a(lds, SET0, ln.w >= 3, ln.w % 3, ln);
    // dE = KI dS_m (+ Aqk^T dO below), own value columns
    f32x4 dE[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x8 sb = pack8(dS[2 * kc], dS[2 * kc + 1]);
#pragma unroll
      for (int I = 0; I < 2; ++I) dE[I] = mma(rd_trp((lb)(lds + O_KI), LT, 32 * kc, 16 * I, ln), sb, dE[I]);
    }
    f32x4 U[2];
    tiles_uw(lds, SET0, U, true, ln);
    __syncthreads();   // #2: A, Aqk, S_m, -W, -U
    ln = fresh();
    {
      const bf16x8 ob = rd_row((lb)(lds + O_DO), LT, 16 * ln.w, 0, ln);
#pragma unroll
      for (int I = 0; I < 2; ++I) dE[I] = mma(rd_row((lb)(lds + O_AQ), LT, 16 * I, 0, ln), ob, dE[I]);
    }
    f32x4 dvv[2];   // dV = beta dY_v, stored with the other gradients
    {
      // dY_v = T^T dE; dV = beta dY_v; dbeta += dY_v . V; dY_v over the own rows of V; -dE
      const bf16x8 eb = pack8(dE[0], dE[1]);
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const f32x4 y = mma(rd_rowp((lb)(lds + O_TT), LT, 16 * I, 0, ln), eb, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 vv = unpack4(ld_raw((lb)(lds + O_V), LT, 16 * ln.w, 16 * I, ln));
        const f32x4 bt = *(const LDS f32x4*)(BETA + 16 * I + 4 * ln.g);
        dvv[I] = bt * y;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = row_sum16(y[r] * vv[r]);
          if (ln.n == 0) DBP[ln.w * BC + 16 * I + 4 * ln.g + r] = s;
        }
        st_t((lb)(lds + O_V), LT, 16 * ln.w, 16 * I, y, ln);
        st_t((lb)(lds + O_NDE), LT, 16 * ln.w, 16 * I, -dE[I], ln);
      }
    }
    // E = U - W S_m -> LDS
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x8 sb = rd_row((lb)(lds + O_R), LR, 16 * ln.w, 32 * kc, ln);
#pragma unroll
      for (int I = 0; I < 2; ++I) U[I] = mma(rd_tr((lb)(lds + O_NW), LT, 32 * kc, 16 * I, ln), sb, U[I]);
    }
#pragma unroll
    for (int I = 0; I < 2; ++I) st_t((lb)(lds + O_E), LT, 16 * ln.w, 16 * I, U[I], ln);
    // own key channels: dQG = dO S_m^T
    f32x4 dQG[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x8 sb = rd_tr((lb)(lds + O_R), LR, 32 * kc, 16 * ln.w, ln);
#pragma unroll
      for (int I = 0; I < 2; ++I) dQG[I] = mma(rd_tr((lb)(lds + O_DO), LT, 32 * kc, 16 * I, ln), sb, dQG[I]);
    }
    __syncthreads();   // #3: -dE, E
    ln = fresh();
    if (m > 0) fetch_s(m - 1, 0, ln);
    // own key channels: dW = -dE S_m^T, dY_k = T^T dW, dKG = beta dY_k, dbeta += dY_k . KG
    f32x4 dKG[2], dYk[2];
    {
      f32x4 dW[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 sb = rd_tr((lb)(lds + O_R), LR, 32 * kc, 16 * ln.w, ln);
#pragma unroll
        for (int I = 0; I < 2; ++I) dW[I] = mma(rd_tr((lb)(lds + O_NDE), LT, 32 * kc, 16 * I, ln), sb, dW[I]);
      }
      const bf16x8 wb = pack8(dW[0], dW[1]);
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        dYk[I] = mma(rd_rowp((lb)(lds + O_TT), LT, 16 * I, 0, ln), wb, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 bt = *(const LDS f32x4*)(BETA + 16 * I + 4 * ln.g);
        const f32x4 kg = unpack4(ld_raw((lb)(lds + O_KG), LT, 16 * ln.w, 16 * I, ln));
        dKG[I] = bt * dYk[I];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = row_sum16(dYk[I][r] * kg[r]);
          if (ln.n == 0) DBP[(NW + ln.w) * BC + 16 * I + 4 * ln.g + r] = s;
        }
      }
    }
    if (ln.w < 3) {
      // dAqk = tril(dO E^T)
      const int I = tile_I(ln.w), J = tile_J(ln.w);
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        acc = mma(rd_tr((lb)(lds + O_DO), LT, 32 * kc, 16 * I, ln),
                  rd_tr((lb)(lds + O_E), LT, 32 * kc, 16 * J, ln), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = (16 * I + 4 * ln.g + r >= 16 * J + ln.n) ? acc[r] : 0.f;
      st_t((lb)(lds + O_DAQ), LT, 16 * J, 16 * I, acc, ln);
    }
    __syncthreads();   // #4: S_m, -dE and dO are done with; dAqk
    ln = fresh();
    if (m > 0) fetch(m - 1, true, ln);
#pragma unroll
    for (int I = 0; I < 2; ++I) st_t((lb)(lds + O_NDE), LT, 16 * ln.w, 16 * I, dYk[I], ln);
    // dS_c = Diag(e^r) (dS_m + QG^T dO - W^T dE); dS_m to R for dKI
    {
      const bf16x8 ob = __builtin_bit_cast(bf16x8, u32x4{o0[0], o0[1], o1[0], o1[1]});
      const bf16x8 eb = pack8(dE[0], dE[1]);
      // the stores first: operand reads that follow no store need not wait on one
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) st_t((lb)(lds + O_R), LR, 16 * ln.w, 16 * cb, dS[cb], ln);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        dS[cb] = mma(rd_rowp((lb)(lds + O_QG), LT, 16 * cb, 0, ln), ob, dS[cb]);
        dS[cb] = mma(rd_rowp((lb)(lds + O_NW), LT, 16 * cb, 0, ln), eb, dS[cb]);
        dS[cb] *= *(const LDS f32x4*)(ER + 16 * cb + 4 * ln.g);
      }
      // keep the operand reads a few products ahead
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    // dQG += dAqk KI; dKI = dAqk^T QG (+ dA^T KG below)
    f32x4 dKI[2];
    {
      const bf16x8 kib = rd_row((lb)(lds + O_KI), LT, 16 * ln.w, 0, ln);
      const bf16x8 qgb = rd_row((lb)(lds + O_QG), LT, 16 * ln.w, 0, ln);
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        dQG[I] = mma(rd_tr((lb)(lds + O_DAQ), LT, 0, 16 * I, ln), kib, dQG[I]);
        dKI[I] = mma(rd_row((lb)(lds + O_DAQ), LT, 16 * I, 0, ln), qgb, f32x4{0.f, 0.f, 0.f, 0.f});
      }
    }
    __syncthreads();   // #5: dY_k, dS_m
    ln = fresh();
    if (m > 0) fetch_s(m - 1, 4, ln);
    if (ln.w < 3) {
      // dL = -(dY_v U^T + dY_k W^T) (strict lower); dbeta += dL . A; dA = Diag(beta) dL
      const int I = tile_I(ln.w), J = tile_J(ln.w);
      f32x4 acc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        acc = mma(rd_tr((lb)(lds + O_V), LT, 32 * kc, 16 * I, ln),
                  rd_tr((lb)(lds + O_NU), LT, 32 * kc, 16 * J, ln), acc);
        acc = mma(rd_tr((lb)(lds + O_NDE), LT, 32 * kc, 16 * I, ln),
                  rd_tr((lb)(lds + O_NW), LT, 32 * kc, 16 * J, ln), acc);
      }
      const LDS float* A = (const LDS float*)(lds + O_A);
      const f32x4 bt = *(const LDS f32x4*)(BETA + 16 * I + 4 * ln.g);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * I + 4 * ln.g + r, j = 16 * J + ln.n;
        acc[r] = i > j ? acc[r] : 0.f;
        const float s = row_sum16(acc[r] * A[i * LA + j]);
        if (ln.n == 0) {
          DBP[(2 * NW + ln.w) * BC + i] = s;
          DBP[(2 * NW + ln.w) * BC + (i ^ 16)] = 0.f;
        }
      }
      st_t((lb)(lds + O_DA), LT, 16 * J, 16 * I, acc * bt, ln);
    }
    // dKIe = E dS_m^T (the K_end part of dKI, kept apart for dlog alpha)
    f32x4 dKIe[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const bf16x8 sb = rd_tr((lb)(lds + O_R), LR, 32 * kc, 16 * ln.w, ln);
#pragma unroll
      for (int I = 0; I < 2; ++I) dKIe[I] = mma(rd_tr((lb)(lds + O_E), LT, 32 * kc, 16 * I, ln), sb, dKIe[I]);
    }
    __syncthreads();   // #6: dA
    ln = fresh();
    {
      const bf16x8 kib = rd_row((lb)(lds + O_KI), LT, 16 * ln.w, 0, ln);
      const bf16x8 kgb = rd_row((lb)(lds + O_KG), LT, 16 * ln.w, 0, ln);
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        dKG[I] = mma(rd_tr((lb)(lds + O_DA), LT, 0, 16 * I, ln), kib, dKG[I]);
        dKI[I] = mma(rd_row((lb)(lds + O_DA), LT, 16 * I, 0, ln), kgb, dKI[I]);
      }
    }
    // epilogue: dq, dk and dlog alpha per element.  The in-chunk pair terms
    // of dlog alpha enter token i (+) and token j (-) of every pair j < i, and
    // the suffix sums cancel those with both tokens at or after t; both sides
    // are formed from the same bf16 factors the products used, so that they
    // cancel to fp32 rounding.  The K_end terms (E dS_m^T) enter as the sum
    // over the tokens before t directly, and the incoming state's decay
    // (sum_v dS_m S_m) enters every token.
    {
      f32x4 db[2], de[2];
      float rs = 0.f;
      for (int p = 0; p < NW; ++p) rs += RP[p * DD + col];
#pragma unroll
      for (int I = 0; I < 2; ++I) {
        const f32x4 qg = unpack4(ld_raw((lb)(lds + O_QG), LT, 16 * ln.w, 16 * I, ln));
        const f32x4 kg = unpack4(ld_raw((lb)(lds + O_KG), LT, 16 * ln.w, 16 * I, ln));
        const f32x4 ki = unpack4(ld_raw((lb)(lds + O_KI), LT, 16 * ln.w, 16 * I, ln));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = __expf(bm[I][r]), pi = __expf(-bm[I][r]);
          db[I][r] = qg[r] * dQG[I][r] + kg[r] * dKG[I][r] - ki[r] * dKI[I][r];
          de[I][r] = ki[r] * dKIe[I][r];
          dQG[I][r] = scale * p * dQG[I][r];
          dKG[I][r] = p * dKG[I][r] + pi * (dKI[I][r] + dKIe[I][r]);
        }
      }
      f32x4 dgc[2];
      suffix_prefix(db, de, dgc, ln);
      dgc[0] += rs;
      dgc[1] += rs;
      store_tile(chunk_view(dq, tok0, L, H, h, DD, 4), dQG, H, ln);
      store_tile(chunk_view(dk, tok0, L, H, h, DD, 4), dKG, H, ln);
      store_tile(chunk_view(dv, tok0, L, H, h, DD, 4), dvv, H, ln);
      if (!SG) store_tile(chunk_view(dg, tok0, L, H, h, DD, 4), dgc, H, ln);
      if (SG) {
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float s = row_sum16(dgc[I][r]);
            if (ln.n == 0) GP[ln.w * BC + 16 * I + 4 * ln.g + r] = s;
          }
      }
    }
    if (m > 0) stage<SG>(lds, xn, true, ln);   // E, -dE and R are done with
    __syncthreads();   // #7: the chunk's LDS may be rewritten
    ln = fresh();
  }
  if (nc > 0) finish_rows(0, ln);
  if (dS0) {
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dS0[sbase + (size_t)(16 * cb + 4 * ln.g + r) * DD + col] = dS[cb][r];
  }
}

}  // namespace

// The poll limit of the forward sweep's tile hand-over: BWD_SPIN, or a
// non-negative count from the environment variable KDA_BWD_SPIN_POLLS (read on
// every call; 0 makes the last wave form every chunk's tiles itself).
constexpr int BWD_SPIN = 512;
static int bwd_spin_polls() {
  const char* e = getenv("KDA_BWD_SPIN_POLLS");
  if (e && *e) {
    char* end = nullptr;
    const long v = strtol(e, &end, 10);
    if (end && *end == '\0' && v >= 0 && v <= BWD_SPIN) return (int)v;
  }
  return BWD_SPIN;
}

hipError_t launch_backward_chunk(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* S0, const void* dout,
                                 const float* dSf, float* dq, float* dk, float* dv, float* dg,
                                 float* dbeta, float* dS0, const int32_t* cu, int n_seq, int T,
                                 int H, float scale, bool scalar_gate, void* states, int* flags,
                                 hipStream_t stream) {
  auto kern = scalar_gate ? bwd_chunk_kernel<true> : bwd_chunk_kernel<false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(n_seq * H), dim3(NT), LDS_BYTES, stream,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, g, beta, S0,
                     (const uint16_t*)dout, dSf, dq, dk, dv, dg, dbeta, dS0, cu, T, H, scale,
                     (uint32_t*)states, flags, bwd_spin_polls());
  return hipGetLastError();
}

}  // namespace kda
