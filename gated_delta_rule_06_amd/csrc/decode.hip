// decode.hip -- the fused recurrent KDA step for one token per sequence.
//
// Schedule: "Kimi Unveils Delta Attention and K3 Architecture Updates",
// section 5 (the fused recurrent kernel): decay the key rows, reduce the
// prediction Sbar^T k, write the outer product k e^T, reduce the read.
// Here the read is fused into the same pass over the state with the algebra
//     o = S_t^T (s q) = s (Sbar^T q + (k^T q) e),
// so each head's fp32 state crosses HBM exactly once in and once out.
//
// Mapping (gfx950, wave64): one 256-thread workgroup per (sequence, head,
// 64-column slice of d_v) -- value columns are independent except for the
// scalar k^T q, which each slice forms itself.  Thread t owns 4 consecutive
// value columns (one float4) of RPT key rows spaced RG apart, so every
// wave-wide load or store covers whole 256-byte runs of the row-major state.
// Splitting the columns halves the state registers per thread (more waves in
// flight per CU; it also narrowed the spread of launch times).  The two
// column reductions go through LDS once.  The state stream is marked
// non-temporal: at 512 MiB it does not fit the last-level cache and is never
// re-read within a step.
#include "common.h"

namespace kda {

// SG: one gate per (sequence, head) for every key row (Gated DeltaNet: log_alpha
// is [N, H]); otherwise one per key row (KDA: [N, H, d_k]).
// FU: the raw inputs pass through the transforms of `pro` (common.h) first.
template <int DK, int DV, class Io, bool SG, bool FU>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ S,
    void* __restrict__ out, float scale, Prologue pro, int H) {
  constexpr int CW = 64;          // value columns per workgroup
  constexpr int NSPLIT = DV / CW;
  constexpr int TPR = CW / 4;     // threads per state row
  constexpr int RG = 256 / TPR;   // row groups
  constexpr int RPT = DK / RG;    // rows per thread
  static_assert(DV % CW == 0 && RPT >= 1 && RG * RPT == DK, "shape");

  const int head = blockIdx.x / NSPLIT;   // n * H + h
  const int c0 = (blockIdx.x % NSPLIT) * CW;
  const int t = threadIdx.x;
  const int cg = t % TPR;
  const int rg = t / TPR;

  __shared__ __attribute__((aligned(16))) float s_k[DK], s_q[DK], s_a[DK];
  __shared__ __attribute__((aligned(16))) float s_p[RG][CW], s_r[RG][CW];
  __shared__ __attribute__((aligned(16))) float s_e[CW];
  __shared__ float s_kq[4], s_k2[4], s_q2[4];

  float* Sh = S + (size_t)head * DK * DV + c0;
  f32x4 st[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    st[m] = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(Sh + (size_t)(rg + RG * m) * DV) + cg);

  // stage this head's k, q and retention factors
  float kq_part = 0.f, k2_part = 0.f, q2_part = 0.f;
  if (t < DK) {
    const size_t i = (size_t)head * DK + t;
    const float kk = Io::load(k, i), qq = Io::load(q, i);
    s_k[t] = kk;
    s_q[t] = qq;
    float gi = SG ? g[head] : g[i];
    if (FU && (pro.flags & PRO_GATE)) {
      const int hh = head % H;
      const float b = pro.bias ? (SG ? pro.bias[hh] : pro.bias[hh * DK + t]) : 0.f;
      gi = gate_logalpha(gi, __expf(pro.A_log[hh]), b);
    }
    s_a[t] = __expf(gi);
    kq_part = kk * qq;
    k2_part = kk * kk;
    q2_part = qq * qq;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) kq_part += __shfl_xor(kq_part, off);
  if ((t & 63) == 0) s_kq[t >> 6] = kq_part;
  if (FU && (pro.flags & PRO_L2NORM)) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      k2_part += __shfl_xor(k2_part, off);
      q2_part += __shfl_xor(q2_part, off);
    }
    if ((t & 63) == 0) {
      s_k2[t >> 6] = k2_part;
      s_q2[t >> 6] = q2_part;
    }
  }
  __syncthreads();
  // L2 norms (FU): the reductions use the raw q and k and are scaled after
  float rk = 1.f, rq = 1.f;
  if (FU && (pro.flags & PRO_L2NORM)) {
    rk = __builtin_amdgcn_rsqf(s_k2[0] + s_k2[1] + s_k2[2] + s_k2[3] + PRO_NORM_EPS);
    rq = __builtin_amdgcn_rsqf(s_q2[0] + s_q2[1] + s_q2[2] + s_q2[3] + PRO_NORM_EPS);
  }

  // forget (decay key rows), then partial prediction and read reductions
  f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    const float a = s_a[row], kk = s_k[row], qq = s_q[row];
    st[m] *= a;
    p += st[m] * kk;
    r += st[m] * qq;
  }
  *reinterpret_cast<f32x4*>(&s_p[rg][4 * cg]) = p;
  *reinterpret_cast<f32x4*>(&s_r[rg][4 * cg]) = r;
  __syncthreads();

  if (t < CW) {
    float pt = 0.f, rt = 0.f;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      pt += s_p[j][t];
      rt += s_r[j][t];
    }
    const float kq = (s_kq[0] + s_kq[1] + s_kq[2] + s_kq[3]) * (rk * rq);
    float b = beta[head];
    if (FU && (pro.flags & PRO_BETA_SIGMOID)) b = sigmoid_f(b);
    const float e = b * (Io::load(v, (size_t)head * DV + c0 + t) - pt * rk);
    s_e[t] = e * rk;                     // the write uses the raw k: k e^T / |k|
    Io::store(out, (size_t)head * DV + c0 + t, scale * (rt * rq + kq * e));
  }
  __syncthreads();

  // write: S = Sbar + k e^T
  const f32x4 e4 = *reinterpret_cast<const f32x4*>(&s_e[4 * cg]);
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int row = rg + RG * m;
    const f32x4 val = st[m] + s_k[row] * e4;
    __builtin_nontemporal_store(val, reinterpret_cast<f32x4*>(Sh + (size_t)row * DV) + cg);
  }
}

template <int DK, int DV, class Io, bool SG, bool FU>
static void launch_dec_k(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float* S, void* out, int NH, int H, float scale,
                         const Prologue& pro, hipStream_t stream) {
  hipLaunchKernelGGL((decode_step_kernel<DK, DV, Io, SG, FU>), dim3(NH * (DV / 64)), dim3(256), 0,
                     stream, q, k, v, g, beta, S, out, scale, pro, H);
}

template <int DK, int DV, class Io>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* g,
                                  const float* beta, float* S, void* out, int NH, int H,
                                  float scale, bool sg, const Prologue& pro, hipStream_t stream) {
  const bool fu = pro.flags != 0;
  if (sg && fu)
    launch_dec_k<DK, DV, Io, true, true>(q, k, v, g, beta, S, out, NH, H, scale, pro, stream);
  else if (sg)
    launch_dec_k<DK, DV, Io, true, false>(q, k, v, g, beta, S, out, NH, H, scale, pro, stream);
  else if (fu)
    launch_dec_k<DK, DV, Io, false, true>(q, k, v, g, beta, S, out, NH, H, scale, pro, stream);
  else
    launch_dec_k<DK, DV, Io, false, false>(q, k, v, g, beta, S, out, NH, H, scale, pro, stream);
  return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float* S, void* out, int NH, int H, int dk, int dv,
                         float scale, bool bf16, bool scalar_gate, const Prologue& pro,
                         hipStream_t stream) {
#define KDA_DEC(DK, DV)                                                                       \
  if (dk == DK && dv == DV)                                                                  \
    return bf16 ? launch_decode_t<DK, DV, IoBf16>(q, k, v, g, beta, S, out, NH, H, scale,      \
                                                  scalar_gate, pro, stream)                  \
                : launch_decode_t<DK, DV, IoF32>(q, k, v, g, beta, S, out, NH, H, scale,       \
                                                 scalar_gate, pro, stream);
  KDA_DEC(64, 64)
  KDA_DEC(64, 128)
  KDA_DEC(128, 64)
  KDA_DEC(128, 128)
#undef KDA_DEC
  return hipErrorInvalidValue;
}

}  // namespace kda
