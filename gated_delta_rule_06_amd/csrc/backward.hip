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
//
// The backward needs the forward states in reverse order.  A forward sweep
// stores the state at the start of every block of BK tokens to the workspace
// (each lane its own registers, so the read back needs no barrier); the
// reverse sweep takes the blocks last to first, and for each token of a block
// recomputes its state from the block's checkpoint (at most BK - 1 forward
// steps) before the backward step.  The token inputs of the current block are
// staged in LDS, two buffers, one barrier per block.
#include "common.h"

namespace kda {

namespace {

constexpr int BK = 4;   // tokens per checkpoint block

template <int DK_, int DV_, class Io_, bool SG_>
struct BwdCfg {
  static constexpr int DK = DK_, DV = DV_;
  typedef Io_ Io;
  static constexpr bool SG = SG_;
  static constexpr int NW = DV / 16;          // waves
  static constexpr int NT = 64 * NW;          // threads
  static constexpr int RPT = DK / 16;         // key rows per lane
  // staged inputs of one block (floats): q, k, g [BK][DK], v, do [BK][DV], beta [BK]
  static constexpr int IN_Q = 0, IN_K = BK * DK, IN_G = 2 * BK * DK, IN_V = 3 * BK * DK;
  static constexpr int IN_DO = IN_V + BK * DV, IN_B = IN_DO + BK * DV;
  static constexpr int IN_SZ = (IN_B + BK + 3) / 4 * 4;
  // per-wave partial sums over the wave's columns: dq, dk, dg [BK][3][NW][DK];
  // dbeta (and the Gated DeltaNet dg) [BK][2][NW]
  static constexpr int RED_SZ = BK * 3 * NW * DK;
  static constexpr int RS_SZ = (BK * 2 * NW + 3) / 4 * 4;
  static constexpr int OFF_IN = 0;
  static constexpr int OFF_RED = OFF_IN + 2 * IN_SZ;
  static constexpr int OFF_RS = OFF_RED + 2 * RED_SZ;
  static constexpr int LDS_FLOATS = OFF_RS + 2 * RS_SZ;
  static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");
};

// Lane coordinates: wave w, row group rg (rows RPT*rg + r), column quad cq
// (columns c0 .. c0 + 3).
struct Lane {
  int w, l, rg, cq, c0;
};

template <class Cfg>
struct Bwd {
  static constexpr int DK = Cfg::DK, DV = Cfg::DV, NW = Cfg::NW, NT = Cfg::NT, RPT = Cfg::RPT;
  typedef typename Cfg::Io Io;

  // The inputs of tokens [tok0, tok0 + L) of head h into one staging buffer
  // (rows past L read as zeros).  Gated DeltaNet gates are copied to every
  // key row.
  static __device__ void stage(float* in, const void* q, const void* k, const void* v,
                               const float* g, const float* beta, const void* dout,
                               size_t tok0, int L, int H, int h) {
    for (int i = threadIdx.x; i < BK * DK; i += NT) {
      const int j = i / DK, c = i - j * DK;
      const size_t e = ((tok0 + j) * H + h) * (size_t)DK + c;
      const bool ok = j < L;
      in[Cfg::IN_Q + i] = ok ? Io::load(q, e) : 0.f;
      in[Cfg::IN_K + i] = ok ? Io::load(k, e) : 0.f;
      in[Cfg::IN_G + i] = ok ? (Cfg::SG ? g[(tok0 + j) * H + h] : g[e]) : 0.f;
    }
    for (int i = threadIdx.x; i < BK * DV; i += NT) {
      const int j = i / DV, c = i - j * DV;
      const size_t e = ((tok0 + j) * H + h) * (size_t)DV + c;
      const bool ok = j < L;
      in[Cfg::IN_V + i] = ok ? Io::load(v, e) : 0.f;
      in[Cfg::IN_DO + i] = ok ? Io::load(dout, e) : 0.f;
    }
    if (threadIdx.x < BK)
      in[Cfg::IN_B + threadIdx.x] = (int)threadIdx.x < L ? beta[(tok0 + threadIdx.x) * H + h] : 0.f;
  }

  // RPT consecutive staged floats (rows RPT*rg ..) into registers
  static __device__ __forceinline__ void rows(const float* p, float (&x)[RPT]) {
#pragma unroll
    for (int i = 0; i < RPT; i += 4) {
      const f32x4 t = *reinterpret_cast<const f32x4*>(p + i);
      x[i] = t[0]; x[i + 1] = t[1]; x[i + 2] = t[2]; x[i + 3] = t[3];
    }
  }

  // One forward step of token j of the staged block on S (in place).
  static __device__ __forceinline__ void fwd_step(f32x4 (&S)[RPT], const float* in, int j,
                                                  const Lane& ln) {
    float kr[RPT], gr[RPT];
    rows(in + Cfg::IN_K + j * DK + RPT * ln.rg, kr);
    rows(in + Cfg::IN_G + j * DK + RPT * ln.rg, gr);
    const f32x4 vv = *reinterpret_cast<const f32x4*>(in + Cfg::IN_V + j * DV + ln.c0);
    const float b = in[Cfg::IN_B + j];
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      S[r] *= __expf(gr[r]);
      p += S[r] * kr[r];
    }
    f32x4 e;
#pragma unroll
    for (int c = 0; c < 4; ++c) e[c] = b * (vv[c] - row_sum16(p[c]));
#pragma unroll
    for (int r = 0; r < RPT; ++r) S[r] += kr[r] * e;
  }

  // Sum over the four column quads of the wave (lanes l, l^16, l^32, l^48).
  static __device__ __forceinline__ float quad_sum(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
  }

  // Token j of the staged block, from its previous state Sp: the forward step
  // it needs (Sbar, p, e, S_j), then the backward step on dS.  Per-wave
  // partials of dq, dk, dg go to red[j], of dbeta (and the Gated DeltaNet dg)
  // to rs[j]; dv is final and goes straight out.
  static __device__ __forceinline__ void bwd_step(const f32x4 (&Sp)[RPT], f32x4 (&dS)[RPT],
                                                  const float* in, int j, float* red, float* rs,
                                                  float* dv_out, float scale, const Lane& ln) {
    float kr[RPT], gr[RPT], qr[RPT];
    rows(in + Cfg::IN_K + j * DK + RPT * ln.rg, kr);
    rows(in + Cfg::IN_G + j * DK + RPT * ln.rg, gr);
    rows(in + Cfg::IN_Q + j * DK + RPT * ln.rg, qr);
    const f32x4 vv = *reinterpret_cast<const f32x4*>(in + Cfg::IN_V + j * DV + ln.c0);
    const f32x4 dov = *reinterpret_cast<const f32x4*>(in + Cfg::IN_DO + j * DV + ln.c0);
    const float b = in[Cfg::IN_B + j];
    // forward: Sbar, p, e
    f32x4 Sb[RPT];
    float a[RPT];
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      a[r] = __expf(gr[r]);
      Sb[r] = Sp[r] * a[r];
      p += Sb[r] * kr[r];
    }
    f32x4 e, vp;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float pc = row_sum16(p[c]);
      vp[c] = vv[c] - pc;
      e[c] = b * vp[c];
    }
    // the read: dS += scale q do^T, dq = scale S_j do (S_j = Sbar + k e^T)
    float dqp[RPT];
    f32x4 de = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const f32x4 Sj = Sb[r] + kr[r] * e;
      const f32x4 t = Sj * dov;
      dqp[r] = scale * ((t[0] + t[1]) + (t[2] + t[3]));
      dS[r] += (scale * qr[r]) * dov;
      de += dS[r] * kr[r];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) de[c] = row_sum16(de[c]);
    const f32x4 dp = -b * de;
    // dbeta over the lane's columns (the same in the 16 lanes of a row group)
    const f32x4 tb = de * vp;
    float dbp = (tb[0] + tb[1]) + (tb[2] + tb[3]);
    float dkp[RPT], dgp[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const f32x4 t = dS[r] * e + Sb[r] * dp;
      dkp[r] = (t[0] + t[1]) + (t[2] + t[3]);
      const f32x4 dSb = dS[r] + kr[r] * dp;
      const f32x4 u = Sb[r] * dSb;
      dgp[r] = (u[0] + u[1]) + (u[2] + u[3]);
      dS[r] = dSb * a[r];
    }
    // dv: final, one lane per column quad
    if (ln.rg == 0) *reinterpret_cast<f32x4*>(dv_out + ln.c0) = b * de;
    // sums over the wave's 16 columns
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      dqp[r] = quad_sum(dqp[r]);
      dkp[r] = quad_sum(dkp[r]);
      dgp[r] = quad_sum(dgp[r]);
    }
    dbp = quad_sum(dbp);
    float* rj = red + j * 3 * NW * DK + ln.w * DK + RPT * ln.rg;
    if (ln.cq == 0) {
#pragma unroll
      for (int r = 0; r < RPT; r += 4) {
        *reinterpret_cast<f32x4*>(rj + r) = f32x4{dqp[r], dqp[r + 1], dqp[r + 2], dqp[r + 3]};
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

  // Sums over the waves of one block's partials, to dq, dk, dg, dbeta.
  static __device__ void write_out(const float* red, const float* rs, size_t tok0, int L, int H,
                                   int h, float* dq, float* dk, float* dg, float* dbeta) {
    for (int i = threadIdx.x; i < L * 3 * DK; i += NT) {
      const int j = i / (3 * DK), rem = i - j * 3 * DK;
      const int qty = rem / DK, row = rem - qty * DK;
      if (Cfg::SG && qty == 2) continue;
      const float* src = red + (j * 3 + qty) * NW * DK + row;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += src[w * DK];
      float* dst = qty == 0 ? dq : (qty == 1 ? dk : dg);
      dst[((tok0 + j) * H + h) * (size_t)DK + row] = s;
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
// DK*DV floats in the lanes' own order.
template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void kda_bwd_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ S0,
    const void* __restrict__ dout, const float* __restrict__ dSf, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ dg,
    float* __restrict__ dbeta, float* __restrict__ dS0, const int32_t* __restrict__ cu, int T,
    int H, float scale, float* __restrict__ ws) {
  typedef Bwd<Cfg> K;
  constexpr int DK = Cfg::DK, DV = Cfg::DV, RPT = Cfg::RPT;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int nh = blockIdx.x, n = nh / H, h = nh - n * H;
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
  const size_t slot_stride = (size_t)H * DK * DV;
  float* ck = ws + ((size_t)n + t0 / BK) * slot_stride + (size_t)h * DK * DV;
  // this lane's float4 of row r inside a checkpoint slot
  auto ck_at = [&](int m, int r) {
    return reinterpret_cast<f32x4*>(ck + m * slot_stride +
                                    (size_t)((ln.w * RPT + r) * 64 + ln.l) * 4);
  };
  const size_t sbase = (size_t)nh * DK * DV + (size_t)(RPT * ln.rg) * DV + ln.c0;

  // forward sweep: checkpoint at the start of every block
  f32x4 S[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    S[r] = S0 ? *reinterpret_cast<const f32x4*>(S0 + sbase + (size_t)r * DV)
              : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int m = 0; m < nb; ++m) {
    const int L = (len - m * BK) < BK ? (len - m * BK) : BK;
    float* in = lds + Cfg::OFF_IN + (m & 1) * Cfg::IN_SZ;
#pragma unroll
    for (int r = 0; r < RPT; ++r) *ck_at(m, r) = S[r];
    K::stage(in, q, k, v, g, beta, dout, t0 + (size_t)m * BK, L, H, h);
    __syncthreads();
    for (int j = 0; j < L; ++j) K::fwd_step(S, in, j, ln);
  }
  __syncthreads();

  // reverse sweep
  f32x4 dS[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
    dS[r] = dSf ? *reinterpret_cast<const f32x4*>(dSf + sbase + (size_t)r * DV)
                : f32x4{0.f, 0.f, 0.f, 0.f};
  for (int m = nb - 1; m >= 0; --m) {
    const int p = m & 1;
    const int L = (len - m * BK) < BK ? (len - m * BK) : BK;
    const size_t tok0 = t0 + (size_t)m * BK;
    float* in = lds + Cfg::OFF_IN + p * Cfg::IN_SZ;
    float* red = lds + Cfg::OFF_RED + p * Cfg::RED_SZ;
    float* rs = lds + Cfg::OFF_RS + p * Cfg::RS_SZ;
    K::stage(in, q, k, v, g, beta, dout, tok0, L, H, h);
    __syncthreads();
    if (m + 1 < nb) {
      const int Ln = (len - (m + 1) * BK) < BK ? (len - (m + 1) * BK) : BK;
      K::write_out(lds + Cfg::OFF_RED + (p ^ 1) * Cfg::RED_SZ,
                   lds + Cfg::OFF_RS + (p ^ 1) * Cfg::RS_SZ, tok0 + BK, Ln, H, h, dq, dk, dg,
                   dbeta);
    }
    f32x4 Sc[RPT];
#pragma unroll
    for (int r = 0; r < RPT; ++r) Sc[r] = *ck_at(m, r);
    for (int j = L - 1; j >= 0; --j) {
      f32x4 Sw[RPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) Sw[r] = Sc[r];
      for (int t = 0; t < j; ++t) K::fwd_step(Sw, in, t, ln);
      K::bwd_step(Sw, dS, in, j, red, rs, dv + ((tok0 + j) * H + h) * (size_t)DV, scale, ln);
    }
  }
  __syncthreads();
  if (nb > 0) {
    const int L0 = len < BK ? len : BK;
    K::write_out(lds + Cfg::OFF_RED, lds + Cfg::OFF_RS, t0, L0, H, h, dq, dk, dg, dbeta);
  }
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
                        hipStream_t stream) {
  const int bytes = Cfg::LDS_FLOATS * 4;
  auto kern = kda_bwd_kernel<Cfg>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(n_seq * H), dim3(Cfg::NT), bytes, stream, q, k, v, g, beta, S0,
                     dout, dSf, dq, dk, dv, dg, dbeta, dS0, cu, T, H, scale, ws);
  return hipGetLastError();
}

}  // namespace

// Checkpoint slots the backward needs: n_seq + rows / BK per head.
size_t backward_workspace_bytes(int n_seq, size_t rows, int H, int dk, int dv) {
  return ((size_t)n_seq + rows / BK) * (size_t)H * dk * dv * sizeof(float);
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* S0, const void* dout, const float* dSf,
                           float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                           const int32_t* cu, int n_seq, int T, int H, int d_k, int d_v,
                           float scale, bool bf16, bool scalar_gate, float* ws,
                           hipStream_t stream) {
#define KDA_BW1(DK, DV, IO, SG)                                                                   \
  return launch_bwd_t<BwdCfg<DK, DV, IO, SG>>(q, k, v, g, beta, S0, dout, dSf, dq, dk, dv, dg,    \
                                              dbeta, dS0, cu, n_seq, T, H, scale, ws, stream);
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
