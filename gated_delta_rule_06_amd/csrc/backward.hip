// backward.hip -- gradients of the KDA forward (training).
//
// The pages give no backward; chunkwise KDA is the training form ("Kimi
// Unveils Delta Attention and K3 Architecture Updates", section 6), so this is
// the reverse-mode derivative of the recurrence of section 4 (forget, predict,
// correct, write, read after the write), step by step in reverse:
//     dS += scale q_t do_t^T;     dq_t = scale S_t do_t
//     de  = dS^T k_t;             dk_t = dS e_t + Sbar_t dp,  dp = -beta_t de
//     dv_t = beta_t de;           dbeta_t = de . (v_t - Sbar_t^T k_t)
//     dSbar = dS + k_t dp^T;      dg_t = rowsum(Sbar_t * dSbar)
//     dS  = Diag(exp g_t) dSbar   (the gradient of S_{t-1})
// with dS starting at dL/dS_final, and dL/dS0 the dS left at the end.
//
// Mapping (gfx950, wave64): one workgroup per (sequence, head) with d_v / 16
// waves; wave w owns value columns [16w, 16w + 16) of every key row, and lane l
// holds rows RPT*(l & 15) .. +RPT-1 of columns 16w + 4*(l >> 4) .. +3 (RPT =
// d_k / 16), of S, of the recomputed states and of dS, all in registers.
// Sums over key rows (p, de) stay inside a 16-lane DPP row; sums over value
// columns (dq, dk, dg, dbeta) take two lane shuffles inside the wave and then
// one LDS slot per wave, added over the waves once per block of BK tokens.
// dq = scale S_t do_t needs only the forward state, so the forward sweep forms
// it; the reverse sweep, which is short of registers, does the rest.
//
// The backward needs the forward states in reverse order.  A forward sweep
// stores the state at the start of every block of BK = 8 tokens to the
// workspace (each lane its own registers, so the read back needs no barrier),
// and v - p of every token.  The reverse sweep takes the blocks last to first;
// the states before a block's tokens 0, 1 and 4 stay in registers, the others
// are recomputed from the nearest one below (13 steps per 8 tokens, each a
// decay and a rank-1 update from the stored v - p, with no reduction).  The
// checkpoints are most of the kernel's memory traffic (d_k d_v fp32 per head
// and block, written once and read once), hence the block length.  A block's
// token inputs are staged in LDS (two buffers); the next block's inputs and
// checkpoint load while this one runs.
#include "common.h"

namespace kda {

namespace {

constexpr int BK = 8;   // tokens per checkpoint block

template <int DK_, int DV_, class Io_, bool SG_>
struct BwdCfg {
  static constexpr int DK = DK_, DV = DV_;
  typedef Io_ Io;
  static constexpr bool SG = SG_;
  static constexpr int NW = DV / 16;          // waves
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int RPT = DK / 16;         // key rows per lane
  // staged inputs of one block (floats): q, k, alpha = exp(g) [BK][DK]; v (forward sweep)
  // or v - p (reverse sweep), do [BK][DV]; beta [BK]
  static constexpr int IN_Q = 0, IN_K = BK * DK, IN_G = 2 * BK * DK, IN_V = 3 * BK * DK;
  static constexpr int IN_DO = IN_V + BK * DV, IN_B = IN_DO + BK * DV;
  static constexpr int IN_SZ = (IN_B + BK + 3) / 4 * 4;
  // staging elements per thread (key-row arrays, value-column arrays)
  static constexpr int NQ = (BK * DK + NT - 1) / NT, NV = (BK * DV + NT - 1) / NT;
  // per-wave partial sums over the wave's columns: dq, dk, dg [BK][3][NW][DK];
  // dbeta (and the Gated DeltaNet dg) [BK][2][NW]
  static constexpr int RED_SZ = BK * 3 * NW * DK;
  static constexpr int RS_SZ = (BK * 2 * NW + 3) / 4 * 4;
  static constexpr int OFF_IN = 0;                  // two staging buffers
  static constexpr int OFF_RED = OFF_IN + 2 * IN_SZ;  // one block of partials
  static constexpr int OFF_RS = OFF_RED + RED_SZ;
  static constexpr int LDS_FLOATS = OFF_RS + RS_SZ;
  static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");
  static_assert(LDS_FLOATS >= KDA_LPT_MAX + 1, "LDS holds the length ranking");
};

// Lane coordinates: wave w, row group rg (rows RPT*rg + r), column quad cq
// (columns c0 .. c0 + 3).
struct Lane {
  int w, l, rg, cq, c0;
};

template <class Cfg>
struct Bwd {
  static constexpr int DK = Cfg::DK, DV = Cfg::DV, NW = Cfg::NW, NT = Cfg::NT, RPT = Cfg::RPT;
  static constexpr int NQ = Cfg::NQ, NV = Cfg::NV;
  typedef typename Cfg::Io Io;

  // One block's inputs in flight, this thread's share: loaded early into
  // registers, written to a staging buffer once the buffer is free.  Rows
  // past the block's length read as zeros.  Gated DeltaNet gates are copied to
  // every key row.  REV: the reverse sweep's set (q, k, g, v - p from the
  // workspace, do, beta); otherwise the forward sweep's (k, g, v, do, beta).
  struct Stage {
    float q[NQ], k[NQ], g[NQ], v[NV], d[NV], b;
  };
  template <bool REV>
  static __device__ __forceinline__ void stage_load(Stage& st, const void* q, const void* k,
                                                    const void* v, const float* g,
                                                    const float* beta, const void* dout,
                                                    const float* vp, size_t tok0, int L, int H,
                                                    int h) {
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const int i = threadIdx.x + s * NT;
      const int j = i / DK, c = i - j * DK;
      const size_t e = ((tok0 + j) * H + h) * (size_t)DK + c;
      const bool ok = i < BK * DK && j < L;
      st.q[s] = (REV && ok) ? Io::load(q, e) : 0.f;
      st.k[s] = ok ? Io::load(k, e) : 0.f;
      st.g[s] = ok ? (Cfg::SG ? g[(tok0 + j) * H + h] : g[e]) : 0.f;
    }
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int i = threadIdx.x + s * NT;
      const int j = i / DV, c = i - j * DV;
      const size_t e = ((tok0 + j) * H + h) * (size_t)DV + c;
      const bool ok = i < BK * DV && j < L;
      st.v[s] = ok ? (REV ? __builtin_nontemporal_load(vp + e) : Io::load(v, e)) : 0.f;
      st.d[s] = ok ? Io::load(dout, e) : 0.f;
    }
    st.b = (int)threadIdx.x < L ? beta[(tok0 + threadIdx.x) * H + h] : 0.f;
  }
  static __device__ __forceinline__ void stage_store(const Stage& st, float* in) {
#pragma unroll
    for (int s = 0; s < NQ; ++s) {
      const int i = threadIdx.x + s * NT;
      if (i < BK * DK) {
        in[Cfg::IN_Q + i] = st.q[s];
        in[Cfg::IN_K + i] = st.k[s];
        in[Cfg::IN_G + i] = __expf(st.g[s]);   // the decay factor alpha
      }
    }
#pragma unroll
    for (int s = 0; s < NV; ++s) {
      const int i = threadIdx.x + s * NT;
      if (i < BK * DV) {
        in[Cfg::IN_V + i] = st.v[s];
        in[Cfg::IN_DO + i] = st.d[s];
      }
    }
    if (threadIdx.x < BK) in[Cfg::IN_B + threadIdx.x] = st.b;
  }

  // RPT consecutive staged floats (rows RPT*rg ..) into registers
  static __device__ __forceinline__ void rows(const float* p, float (&x)[RPT]) {
#pragma unroll
    for (int i = 0; i < RPT; i += 4) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(p + i);
      x[i] = t[0]; x[i + 1] = t[1]; x[i + 2] = t[2]; x[i + 3] = t[3];
    }
  }

  // Sum over the four column quads of the wave (lanes l, l^16, l^32, l^48).
  static __device__ __forceinline__ float quad_sum(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
  }

  // Forward sweep, token j of the staged block: the full step on S; v - p of
  // the lane's columns to `vp_out` (one lane per column quad); and the wave's
  // part of dq_j = scale S_j do_j (S_j after the write: the read of the forward
  // needs no backward quantity) to `red_j`.
  static __device__ __forceinline__ void fwd_step(f32x4 (&S)[RPT], const float* in, int j,
                                                  float* vp_out, float* red_j, float scale,
                                                  const Lane& ln) {
    float kr[RPT], gr[RPT];
    rows(in + Cfg::IN_K + j * DK + RPT * ln.rg, kr);
    rows(in + Cfg::IN_G + j * DK + RPT * ln.rg, gr);
    const f32x4 vv = *reinterpret_cast<const f32x4*>(in + Cfg::IN_V + j * DV + ln.c0);
    const float b = in[Cfg::IN_B + j];
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      S[r] *= gr[r];
      p += S[r] * kr[r];
    }
    f32x4 vp;
#pragma unroll
    for (int c = 0; c < 4; ++c) vp[c] = vv[c] - row_sum16(p[c]);
    if (ln.rg == 0) __builtin_nontemporal_store(vp, reinterpret_cast<f32x4*>(vp_out + ln.c0));
    const f32x4 e = b * vp;
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] += kr[r] * e;
    const f32x4 dov = *reinterpret_cast<const f32x4*>(in + Cfg::IN_DO + j * DV + ln.c0);
    float dqp[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      float t = S[r][0] * dov[0];
      t = __builtin_fmaf(S[r][1], dov[1], t);
      t = __builtin_fmaf(S[r][2], dov[2], t);
      t = __builtin_fmaf(S[r][3], dov[3], t);
      dqp[r] = scale * quad_sum(t);
    }
    if (ln.cq == 0) {
      float* rj = red_j + ln.w * DK + RPT * ln.rg;
#pragma unroll
      for (int r = 0; r < RPT; r += 4)
        *reinterpret_cast<f32x4*>(rj + r) = f32x4{dqp[r], dqp[r + 1], dqp[r + 2], dqp[r + 3]};
    }
  }

  // Reverse sweep, recomputing: the step of token j from the stored v - p
  // (no reduction).
  static __device__ __forceinline__ void re_step(f32x4 (&S)[RPT], const float* in, int j,
                                                 const Lane& ln) {
    float kr[RPT], gr[RPT];
    rows(in + Cfg::IN_K + j * DK + RPT * ln.rg, kr);
    rows(in + Cfg::IN_G + j * DK + RPT * ln.rg, gr);
    const f32x4 e = in[Cfg::IN_B + j] * *reinterpret_cast<const f32x4*>(in + Cfg::IN_V + j * DV + ln.c0);
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] = S[r] * gr[r] + kr[r] * e;
  }


  // Token j of the staged block, from its previous state Sp: the backward
  // step on dS.  Per-wave partials of dk, dg go to red[j], of dbeta (and the
  // Gated DeltaNet dg) to rs[j]; dv is final and goes straight out.  (dq came
  // from the forward sweep.)
  static __device__ __forceinline__ void bwd_step(const f32x4 (&Sp)[RPT], f32x4 (&dS)[RPT],
                                                  const float* in, int j, float* red, float* rs,
                                                  float* dv_out, float scale, const Lane& ln) {
    float kr[RPT], gr[RPT], qr[RPT];
    rows(in + Cfg::IN_K + j * DK + RPT * ln.rg, kr);
    rows(in + Cfg::IN_G + j * DK + RPT * ln.rg, gr);
    rows(in + Cfg::IN_Q + j * DK + RPT * ln.rg, qr);
    const f32x4 vp = *reinterpret_cast<const f32x4*>(in + Cfg::IN_V + j * DV + ln.c0);
    const f32x4 dov = *reinterpret_cast<const f32x4*>(in + Cfg::IN_DO + j * DV + ln.c0);
    const float b = in[Cfg::IN_B + j];
    const f32x4 e = b * vp;
    // the read o = scale S_j^T q: dS += scale q do^T
    const float (&a)[RPT] = gr;
    f32x4 de = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      dS[r] += (scale * qr[r]) * dov;
      de += dS[r] * kr[r];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) de[c] = row_sum16(de[c]);
    const f32x4 dp = -b * de;
    // dbeta over the lane's columns (the same in the 16 lanes of a row group)
    float dbp = de[0] * vp[0] + de[1] * vp[1] + de[2] * vp[2] + de[3] * vp[3];
    float dkp[RPT], dgp[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const f32x4 Sb = Sp[r] * a[r];   // Sbar = Diag(alpha) Sp
      float x = dS[r][0] * e[0];
      x = __builtin_fmaf(dS[r][1], e[1], x);
      x = __builtin_fmaf(dS[r][2], e[2], x);
      x = __builtin_fmaf(dS[r][3], e[3], x);
      x = __builtin_fmaf(Sb[0], dp[0], x);
      x = __builtin_fmaf(Sb[1], dp[1], x);
      x = __builtin_fmaf(Sb[2], dp[2], x);
      dkp[r] = __builtin_fmaf(Sb[3], dp[3], x);
      const f32x4 dSb = dS[r] + kr[r] * dp;
      float y = Sb[0] * dSb[0];
      y = __builtin_fmaf(Sb[1], dSb[1], y);
      y = __builtin_fmaf(Sb[2], dSb[2], y);
      dgp[r] = __builtin_fmaf(Sb[3], dSb[3], y);
      dS[r] = dSb * a[r];
    }
    // dv: final, one lane per column quad
    if (ln.rg == 0) __builtin_nontemporal_store(b * de, reinterpret_cast<f32x4*>(dv_out + ln.c0));
    // sums over the wave's 16 columns
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      dkp[r] = quad_sum(dkp[r]);
      dgp[r] = quad_sum(dgp[r]);
    }
    dbp = quad_sum(dbp);
    float* rj = red + j * 3 * NW * DK + ln.w * DK + RPT * ln.rg;
    if (ln.cq == 0) {
#pragma unroll
      for (int r = 0; r < RPT; r += 4) {
        *reinterpret_cast<f32x4*>(rj + NW * DK + r) =
            f32x4{dkp[r], dkp[r + 1], dkp[r + 2], dkp[r + 3]};
        if (!Cfg::SG)
          *reinterpret_cast<f32x4*>(rj + 2 * NW * DK + r) =
              f32x4{dgp[r], dgp[r + 1], dgp[r + 2], dgp[r + 3]};
      }
    }
    float* sj = rs + j * 2 * NW + ln.w;
    if (Cfg::SG) {
      // one gate for every row: the sum over the wave's rows as well
      float x = 0.f;
#pragma unroll
      for (int r = 0; r < RPT; ++r) x += dgp[r];
      x = row_sum16(x);
      if (ln.l == 0) sj[NW] = x;
    }
    if (ln.l == 0) sj[0] = dbp;
  }

  // Sums over the waves of one block's dq partials (slot `slot` of red).
  static __device__ void write_dq(const float* red, int slot, size_t tok0, int L, int H, int h,
                                  float* dq) {
    for (int i = threadIdx.x; i < L * DK; i += NT) {
      const int j = i / DK, row = i - j * DK;
      const float* src = red + (j * 3 + slot) * NW * DK + row;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += src[w * DK];
      __builtin_nontemporal_store(s, dq + ((tok0 + j) * H + h) * (size_t)DK + row);
    }
  }

  // Sums over the waves of one block's partials, to dk, dg (slots 1, 2), dbeta.
  static __device__ void write_out(const float* red, const float* rs, size_t tok0, int L, int H,
                                   int h, float* dk, float* dg, float* dbeta) {
    for (int i = threadIdx.x; i < L * 2 * DK; i += NT) {
      const int j = i / (2 * DK), rem = i - j * 2 * DK;
      const int qty = 1 + rem / DK, row = rem - (qty - 1) * DK;
      if (Cfg::SG && qty == 2) continue;
      const float* src = red + (j * 3 + qty) * NW * DK + row;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += src[w * DK];
      float* dst = qty == 1 ? dk : dg;
      __builtin_nontemporal_store(s, dst + ((tok0 + j) * H + h) * (size_t)DK + row);
    }
    if ((int)threadIdx.x < L) {
      const int j = threadIdx.x;
      float sb = 0.f, sg = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sb += rs[j * 2 * NW + w];
        sg += rs[j * 2 * NW + NW + w];
      }
      dbeta[(tok0 + j) * H + h] = sb;
      if (Cfg::SG) dg[(tok0 + j) * H + h] = sg;
    }
  }
};

// S0, dS_final, dS0 are [n_seq, H, DK, DV].  ws holds the checkpoints: for
// sequence n (first token t0), block m of head h is slot (n + t0/BK + m)*H + h,
// DK*DV floats in the lanes' own order; after them, vp [rows, H, DV] holds
// v - p of every token (p = Sbar^T k, from the forward sweep).
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void kda_bwd_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ S0,
    const void* __restrict__ dout, const float* __restrict__ dSf, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta, float* __restrict__ dS0, const int32_t* __restrict__ cu, int T,
    int H, float scale, float* ws, float* vp, const int* __restrict__ only) {
  typedef Bwd<Cfg> K;
  typedef typename K::Stage Stage;
  constexpr int DK = Cfg::DK, DV = Cfg::DV, RPT = Cfg::RPT;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  // Packed sequences: workgroup b takes head b % H of the (b / H)-th longest
  // sequence (ties by index; each workgroup ranks the lengths itself in LDS,
  // up to KDA_LPT_MAX sequences), so that long chains start first.
  const int h = blockIdx.x % H;
  int n = blockIdx.x / H;
  if (cu && (int)(gridDim.x / H) <= KDA_LPT_MAX) {
    const int N = gridDim.x / H;
    int* lens = reinterpret_cast<int*>(lds);
    int* sel = lens + KDA_LPT_MAX;
    for (int m = threadIdx.x; m < N; m += Cfg::NT) lens[m] = cu[m + 1] - cu[m];
    __syncthreads();
    for (int m = threadIdx.x; m < N; m += Cfg::NT) {
      const int lm = lens[m];
      int rank = 0;
      for (int j = 0; j < N; ++j) rank += (lens[j] > lm) || (lens[j] == lm && j < m);
      if (rank == n) *sel = m;
    }
    __syncthreads();
    n = *sel;
    __syncthreads();   // the LDS is the kernel's from here on
  }
  const int nh = n * H + h;
  if (only && only[nh] == 0) return;   // a chain the chunkwise backward has done
  Lane ln;
  ln.w = threadIdx.x >> 6;
  ln.l = threadIdx.x & 63;
  ln.rg = ln.l & 15;
  ln.cq = ln.l >> 4;
  ln.c0 = 16 * ln.w + 4 * ln.cq;
  size_t t0;
  int len;
  if (cu) {
    t0 = (size_t)cu[n];
    len = cu[n + 1] - cu[n];
  } else {
    t0 = (size_t)n * T;
    len = T;
  }
  const int nb = (len + BK - 1) / BK;
  auto blen = [&](int m) { return (len - m * BK) < BK ? (len - m * BK) : BK; };
  const size_t slot_stride = (size_t)H * DK * DV;
  float* ck = ws + ((size_t)n + t0 / BK) * slot_stride + (size_t)h * DK * DV;
  // this lane's float4 of row r inside a checkpoint slot
  auto ck_at = [&](int m, int r) {
    return reinterpret_cast<f32x4*>(ck + m * slot_stride +
                                    (size_t)((ln.w * RPT + r) * 64 + ln.l) * 4);
  };
  auto in_buf = [&](int m) { return lds + Cfg::OFF_IN + (m & 1) * Cfg::IN_SZ; };
  const size_t sbase = (size_t)nh * DK * DV + (size_t)(RPT * ln.rg) * DV + ln.c0;
  float* red = lds + Cfg::OFF_RED;
  float* rs = lds + Cfg::OFF_RS;
  Stage st;

  // forward sweep: checkpoint at the start of every block, v - p per token;
  // the next block's inputs load while this one is computed
  f32x4 S[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    S[r] = S0 ? *reinterpret_cast<const f32x4*>(S0 + sbase + (size_t)r * DV)
              : f32x4{0.f, 0.f, 0.f, 0.f};
  // the inputs of two blocks ahead are in flight, in two register sets that
  // alternate (the loop body is written out twice so that no set is copied)
  Stage sa;
  if (nb > 0) {
    K::template stage_load<false>(st, q, k, v, g, beta, dout, vp, t0, blen(0), H, h);
    K::stage_store(st, in_buf(0));
  }
  if (nb > 1) K::template stage_load<false>(sa, q, k, v, g, beta, dout, vp, t0 + BK, blen(1), H, h);
  auto fwd_block = [&](int m, Stage& next, Stage& later) {
    const int L = blen(m);
    const size_t tok0 = t0 + (size_t)m * BK;
    float* in = in_buf(m);
#pragma unroll
    for (int r = 0; r < RPT; ++r) __builtin_nontemporal_store(S[r], ck_at(m, r));
    __syncthreads();
    // dq of the previous block (its partials in slot (m - 1) & 1; this block
    // writes the other slot, and the next barrier separates the two uses)
    if (m > 0) K::write_dq(red, (m - 1) & 1, tok0 - BK, BK, H, h, dq);
    if (m + 2 < nb)
      K::template stage_load<false>(later, q, k, v, g, beta, dout, vp, tok0 + 2 * BK, blen(m + 2),
                                    H, h);
    auto step = [&](int j) {
      K::fwd_step(S, in, j, vp + ((tok0 + j) * H + h) * (size_t)DV,
                  red + (j * 3 + (m & 1)) * Cfg::NW * DK, scale, ln);
    };
    if (L == BK) {
      // a full block, written out so that one token's dq tail (lane swaps
      // and LDS writes, off the state's dependency chain) overlaps the next
      // token's step
#pragma unroll
      for (int j = 0; j < BK; ++j) step(j);
    } else {
      for (int j = 0; j < L; ++j) step(j);
    }
    if (m + 1 < nb) K::stage_store(next, in_buf(m + 1));
  };
  for (int m = 0; m < nb; m += 2) {
    fwd_block(m, sa, st);
    if (m + 1 < nb) fwd_block(m + 1, st, sa);
  }
  __syncthreads();   // the forward sweep's staging reads and vp writes are done
  if (nb > 0) K::write_dq(red, (nb - 1) & 1, t0 + (size_t)(nb - 1) * BK, blen(nb - 1), H, h, dq);

  // reverse sweep
  f32x4 dS[RPT], Sc[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    dS[r] = dSf ? *reinterpret_cast<const f32x4*>(dSf + sbase + (size_t)r * DV)
                : f32x4{0.f, 0.f, 0.f, 0.f};
  if (nb > 0) {
    K::template stage_load<true>(st, q, k, v, g, beta, dout, vp, t0 + (size_t)(nb - 1) * BK,
                                 blen(nb - 1), H, h);
#pragma unroll
    for (int r = 0; r < RPT; ++r) Sc[r] = __builtin_nontemporal_load(ck_at(nb - 1, r));
    K::stage_store(st, in_buf(nb - 1));
  }
  for (int m = nb - 1; m >= 0; --m) {
    const int L = blen(m);
    const size_t tok0 = t0 + (size_t)m * BK;
    float* in = in_buf(m);
    __syncthreads();   // this block's inputs are staged; the partials hold block m + 1's
    if (m + 1 < nb) {
      K::write_out(red, rs, tok0 + BK, blen(m + 1), H, h, dk, dg, dbeta);
      __syncthreads();   // the partials are free again
    }
    auto dvp = [&](int j) { return dv + ((tok0 + j) * H + h) * (size_t)DV; };
    // States before tokens 0, 1 and 4 of the block stay in registers (Sc, S1,
    // S4); the others are recomputed from the nearest one below: 13 steps for
    // 8 tokens.
    f32x4 S1[RPT], S4[RPT];
    if (L >= 2) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) S1[r] = Sc[r];
      K::re_step(S1, in, 0, ln);
    }
    if (L >= 5) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) S4[r] = S1[r];
      for (int t = 1; t < 4; ++t) K::re_step(S4, in, t, ln);
      for (int j = L - 1; j >= 5; --j) {
        f32x4 Sw[RPT];
#pragma unroll
        for (int r = 0; r < RPT; ++r) Sw[r] = S4[r];
        for (int t = 4; t < j; ++t) K::re_step(Sw, in, t, ln);
        K::bwd_step(Sw, dS, in, j, red, rs, dvp(j), scale, ln);
      }
      K::bwd_step(S4, dS, in, 4, red, rs, dvp(4), scale, ln);
    }
    for (int j = (L < 4 ? L : 4) - 1; j >= 2; --j) {
      f32x4 Sw[RPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) Sw[r] = S1[r];
      for (int t = 1; t < j; ++t) K::re_step(Sw, in, t, ln);
      K::bwd_step(Sw, dS, in, j, red, rs, dvp(j), scale, ln);
    }
    // the previous block's inputs and checkpoint load during the last two tokens
    f32x4 Sn[RPT];
    if (m > 0) {
      K::template stage_load<true>(st, q, k, v, g, beta, dout, vp, tok0 - BK, BK, H, h);
#pragma unroll
      for (int r = 0; r < RPT; ++r) Sn[r] = __builtin_nontemporal_load(ck_at(m - 1, r));
    }
    if (L >= 2) K::bwd_step(S1, dS, in, 1, red, rs, dvp(1), scale, ln);
    K::bwd_step(Sc, dS, in, 0, red, rs, dvp(0), scale, ln);
    if (m > 0) {
#pragma unroll
      for (int r = 0; r < RPT; ++r) Sc[r] = Sn[r];
      K::stage_store(st, in_buf(m - 1));
    }
  }
  __syncthreads();
  if (nb > 0) K::write_out(red, rs, t0, blen(0), H, h, dk, dg, dbeta);
  if (dS0) {
#pragma unroll
    for (int r = 0; r < RPT; ++r) *reinterpret_cast<f32x4*>(dS0 + sbase + (size_t)r * DV) = dS[r];
  }
}

template <class Cfg>
hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* S0, const void* dout, const float* dSf,
                        float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                        const int32_t* cu, int n_seq, int T, int H, float scale, float* ws,
                        const int* only, hipStream_t stream) {
  const int bytes = Cfg::LDS_FLOATS * 4;
  auto kern = kda_bwd_kernel<Cfg>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     bytes);
  if (e != hipSuccess) return e;
  // v - p follows the checkpoint slots (T is T_total when packed)
  const size_t rows = cu ? (size_t)T : (size_t)n_seq * T;
  float* vp = ws + ((size_t)n_seq + rows / BK) * (size_t)H * Cfg::DK * Cfg::DV;
  hipLaunchKernelGGL(kern, dim3(n_seq * H), dim3(Cfg::NT), bytes, stream, q, k, v, g, beta, S0,
                     dout, dSf, dq, dk, dv, dg, dbeta, dS0, cu, T, H, scale, ws, vp, only);
  return hipGetLastError();
}

// One int per chain at the front of the workspace: set by the chunkwise
// backward for chains it leaves to the token loop.
size_t flag_bytes(int n_seq, int H) { return ((size_t)n_seq * H * 4 + 255) / 256 * 256; }

}  // namespace

// The chain flags, then checkpoint slots (n_seq + rows / BK per head) and v - p
// of every token.  The chunkwise backward's states (one bf16 state per 32
// tokens) fit in the space of the checkpoints.
size_t backward_workspace_bytes(int n_seq, size_t rows, int H, int dk, int dv) {
  return flag_bytes(n_seq, H) +
         (((size_t)n_seq + rows / BK) * (size_t)H * dk * dv + rows * (size_t)H * dv) *
             sizeof(float);
}

hipError_t launch_backward_chunk(const void* q, const void* k, const void* v, const float* g,
                                 const float* beta, const float* S0, const void* dout,
                                 const float* dSf, float* dq, float* dk, float* dv, float* dg,
                                 float* dbeta, float* dS0, const int32_t* cu, int n_seq, int T,
                                 int H, float scale, bool scalar_gate, void* states, int* flags,
                                 hipStream_t stream);

hipError_t launch_backward(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* S0, const void* dout, const float* dSf,
                           float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                           const int32_t* cu, int n_seq, int T, int H, int d_k, int d_v,
                           float scale, bool bf16, bool scalar_gate, float* ws,
                           hipStream_t stream) {
  // bf16 at d_k = d_v = 128: the chunkwise backward on MFMA, then the token
  // loop for the chains it flagged (a chunk whose decay is beyond its range)
  int* flags = reinterpret_cast<int*>(ws);
  const int* only = nullptr;
  ws = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + flag_bytes(n_seq, H));
  if (bf16 && d_k == 128 && d_v == 128) {
    const hipError_t e =
        launch_backward_chunk(q, k, v, g, beta, S0, dout, dSf, dq, dk, dv, dg, dbeta, dS0, cu,
                              n_seq, T, H, scale, scalar_gate, ws, flags, stream);
    if (e != hipSuccess) return e;
    only = flags;
  }
#define KDA_BW1(DK, DV, IO, SG)                                                                   \
  return launch_bwd_t<BwdCfg<DK, DV, IO, SG>>(q, k, v, g, beta, S0, dout, dSf, dq, dk, dv, dg,    \
                                              dbeta, dS0, cu, n_seq, T, H, scale, ws, only,       \
                                              stream);
#define KDA_BW(DK, DV)                                      \
  if (bf16) {                                               \
    if (scalar_gate) { KDA_BW1(DK, DV, IoBf16, true) }      \
    KDA_BW1(DK, DV, IoBf16, false)                          \
  }                                                         \
  if (scalar_gate) { KDA_BW1(DK, DV, IoF32, true) }         \
  KDA_BW1(DK, DV, IoF32, false)
  if (d_k == 128 && d_v == 128) { KDA_BW(128, 128) }
  if (d_k == 128 && d_v == 64) { KDA_BW(128, 64) }
  if (d_k == 64 && d_v == 128) { KDA_BW(64, 128) }
  if (d_k == 64 && d_v == 64) { KDA_BW(64, 64) }
#undef KDA_BW
#undef KDA_BW1
  return hipErrorInvalidValue;
}

}  // namespace kda
