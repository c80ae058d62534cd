// recurrent.hip -- the fused recurrent KDA form over several tokens per
// sequence (multi-token decode, speculative verification, short prefill).
//
// The recurrence itself ("Kimi Unveils Delta Attention and K3 Architecture
// Updates", section 5, the fused recurrent kernel, whose regime is decode,
// short sequences and stateful serving; "Linear Attention, From Scratch to
// Kimi 3", section 6 for the recurrence and section 9, where the fused kernel
// loops over several tokens), token by token on a state that stays in
// registers from the sequence's first token to its last:
//     Sbar = Diag(exp(g_t)) S,  e = beta_t (v_t - Sbar^T k_t),
//     S <- Sbar + k_t e^T,      o_t = scale (Sbar^T q_t + (k_t^T q_t) e)
// (the read o_t = S_t^T (scale q_t), expanded so that both reductions use the
// decayed state of the same pass).  The state crosses HBM once in and once
// out per call, however many tokens the sequence has.
//
// Mapping (gfx950, wave64): one 256-thread workgroup per (sequence, head,
// 64-column slice of d_v); each wave owns 16 value columns and all d_k key
// rows of them, so a wave needs no barrier and no LDS.  Lane l holds rows
// RPT*(l & 15) .. RPT*(l & 15) + RPT - 1 of columns 4*(l >> 4) .. +3 (RPT =
// d_k / 16 float4 registers): the reductions over key rows stay inside each
// 16-lane DPP row (four rotate-and-add steps), and every lane ends with the
// complete sums.  The next token's inputs are loaded while the current one is
// processed.
#include "common.h"

namespace kda {

namespace {

// N consecutive elements of one token row, as raw dwords.
template <class Io, int N>
struct RowVec {
  static constexpr int NW = Io::is_bf16 ? N / 2 : N;
  static_assert(NW == 2 || NW % 4 == 0, "row vector size");
  uint32_t w[NW];
  __device__ __forceinline__ void load(const void* base, size_t elem) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(
        reinterpret_cast<const char*>(base) + elem * sizeof(typename Io::storage));
    if constexpr (NW == 2) {
      const u32x2 x = *reinterpret_cast<const u32x2*>(p);
      w[0] = x[0];
      w[1] = x[1];
    } else {
#pragma unroll
      for (int i = 0; i < NW; i += 4) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(p + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) w[i + j] = x[j];
      }
    }
  }
  __device__ __forceinline__ float get(int i) const {
    if (Io::is_bf16)
      return __uint_as_float((i & 1) ? (w[i >> 1] & 0xffff0000u) : (w[i >> 1] << 16));
    return __uint_as_float(w[i]);
  }
};

}  // namespace

// One token's inputs for one lane.  SG: one gate per (token, head) for every
// key row (Gated DeltaNet); otherwise one per key row (KDA).
template <int DK, int DV, class Io, bool SG>
struct RecurrentToken {
  static constexpr int RPT = DK / 16;
  RowVec<Io, RPT> k, q;
  RowVec<IoF32, RPT> g;
  float gs;
  RowVec<Io, 4> v;
  float beta;
  __device__ __forceinline__ void load(const void* qp, const void* kp, const void* vp,
                                       const float* gp, const float* bp, size_t e, int row0,
                                       int col) {
    k.load(kp, e * DK + row0);
    q.load(qp, e * DK + row0);
    if constexpr (SG)
      gs = gp[e];
    else
      g.load(gp, e * DK + row0);
    v.load(vp, e * DV + col);
    beta = bp[e];
  }
  __device__ __forceinline__ float gate(int m) const { return SG ? gs : g.get(m); }
};

// S0 and S_final may be the same array (each workgroup reads its slice of the
// state before it writes it), so neither is marked restrict.
// FU: the raw inputs pass through the transforms of `pro` (common.h) first.
template <int DK, int DV, class Io, bool SG, bool FU>
__global__ __launch_bounds__(256) void recurrent_fwd_kernel(
    const void* __restrict__ q, const void* __restrict__ k, const void* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* S0,
    void* __restrict__ out, float* S_final, const int32_t* __restrict__ cu_seqlens, int T, int H,
    float scale, Prologue pro) {
  constexpr int CW = 64;                 // value columns per workgroup
  constexpr int NSL = DV / CW;
  constexpr int RPT = DK / 16;           // key rows per lane
  // LDS tile of the state slice: rows of CW floats with no padding (32 KB at
  // d_k = 128, so five workgroups fit a CU); the 16-byte slots of a row are
  // XOR-swizzled by the row's lane group (row / RPT), which keeps both the
  // row-wise copies (16 threads per row) and the compute layout's reads (16
  // lanes, one row group each) free of bank conflicts.
  constexpr int LDX = CW;
  constexpr int RSH = RPT == 8 ? 3 : 2;  // log2(RPT)
  static_assert(DV % CW == 0 && DK % 16 == 0, "shape");

  const int slice = blockIdx.x % NSL;
  const int nh = blockIdx.x / NSL;       // n * H + h
  const int n = nh / H, h = nh - n * H;
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int rg = l & 15, cg = l >> 4;
  const int row0 = RPT * rg;
  const int col = slice * CW + w * 16 + 4 * cg;
  int t0, t1;
  if (cu_seqlens) {
    t0 = cu_seqlens[n];
    t1 = cu_seqlens[n + 1];
  } else {
    t0 = n * T;
    t1 = t0 + T;
  }

  // The state slice goes through LDS on its way in and out, so that global
  // memory sees whole 256-byte row segments (16 threads per row, float4
  // each) while the compute layout keeps 16 columns per wave.
  __shared__ __attribute__((aligned(16))) float X[DK * LDX];
  const float* Sg0 = S0 + (size_t)nh * DK * DV + slice * CW;
  const int c4 = 4 * (threadIdx.x & 15), r16 = threadIdx.x >> 4;
  auto xs = [](int row, int col) { return row * LDX + (((col >> 2) ^ ((row >> RSH) & 15)) << 2); };
  float* xl = X + xs(row0, w * 16 + 4 * cg);        // this lane's rows in the compute layout
  f32x4 st[RPT];
  if (S0) {
#pragma unroll
    for (int j = 0; j < DK / 16; ++j) {
      const int row = r16 + 16 * j;
      *reinterpret_cast<f32x4*>(X + xs(row, c4)) =
          __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sg0 + (size_t)row * DV + c4));
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] = *reinterpret_cast<const f32x4*>(xl + m * LDX);
  } else {
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // transform parameters of this head (FU): exp(A_log) and the lane's biases
  float ea = 1.f, gb[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) gb[m] = 0.f;
  if (FU && (pro.flags & PRO_GATE)) {
    ea = __expf(pro.A_log[h]);
    if (pro.bias) {
#pragma unroll
      for (int m = 0; m < RPT; ++m) gb[m] = SG ? pro.bias[h] : pro.bias[h * DK + row0 + m];
    }
  }

  // one token: forget, predict, correct, write, read
  auto token = [&](const RecurrentToken<DK, DV, Io, SG>& in, int t) {
    float kk[RPT], qq[RPT];
    float kq = 0.f, k2 = 0.f, q2 = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      kk[m] = in.k.get(m);
      qq[m] = in.q.get(m);
      kq += kk[m] * qq[m];
      if (FU) {
        k2 += kk[m] * kk[m];
        q2 += qq[m] * qq[m];
      }
    }
    // decay the key rows, then the partial prediction Sbar^T k and read Sbar^T q
    f32x4 p = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
      float gm = in.gate(m);
      if (FU && (pro.flags & PRO_GATE)) gm = gate_logalpha(gm, ea, gb[m]);
      st[m] *= __expf(gm);
      p += st[m] * kk[m];
      r += st[m] * qq[m];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      p[c] = row_sum16(p[c]);
      r[c] = row_sum16(r[c]);
    }
    kq = row_sum16(kq);
    float b = in.beta;
    // L2 norms: the sums above used the raw q and k; scale them afterwards
    // (p by 1/|k|, r by 1/|q|, k^T q by both) and write k e^T as raw k times
    // e/|k|
    float rk = 1.f;
    if (FU) {
      if (pro.flags & PRO_L2NORM) {
        rk = __builtin_amdgcn_rsqf(row_sum16(k2) + PRO_NORM_EPS);
        const float rq = __builtin_amdgcn_rsqf(row_sum16(q2) + PRO_NORM_EPS);
        p *= rk;
        r *= rq;
        kq *= rk * rq;
      }
      if (pro.flags & PRO_BETA_SIGMOID) b = sigmoid_f(b);
    }
    const f32x4 vv = {in.v.get(0), in.v.get(1), in.v.get(2), in.v.get(3)};
    const f32x4 e = b * (vv - p);
    if (rg == 0) Io::store4(out, ((size_t)t * H + h) * DV + col, scale * (r + kq * e));
    // S = Sbar + k e^T
    const f32x4 ek = e * rk;
#pragma unroll
    for (int m = 0; m < RPT; ++m) st[m] += kk[m] * ek;
  };
  auto fetch = [&](RecurrentToken<DK, DV, Io, SG>& in, int t) {
    in.load(q, k, v, g, beta, (size_t)t * H + h, row0, col);
  };

  // Two input buffers, alternating: the loads of token t + 1 are in flight
  // while token t is processed.  The prefetch past the end re-reads the last
  // token, so the loads need no branch.
  if (t0 < t1) {
    RecurrentToken<DK, DV, Io, SG> a, b;
    fetch(a, t0);
    int t = t0;
    for (; t + 1 < t1; t += 2) {
      fetch(b, t + 1);
      token(a, t);
      fetch(a, (t + 2 < t1) ? t + 2 : t + 1);
      token(b, t + 1);
    }
    if (t < t1) token(a, t);
  }

  if (S_final) {
    // each lane overwrites exactly the LDS words it read, so only the
    // transposed read-out needs a barrier
#pragma unroll
    for (int m = 0; m < RPT; ++m) *reinterpret_cast<f32x4*>(xl + m * LDX) = st[m];
    __syncthreads();
    float* Sg1 = S_final + (size_t)nh * DK * DV + slice * CW;
#pragma unroll
    for (int j = 0; j < DK / 16; ++j) {
      const int row = r16 + 16 * j;
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(X + xs(row, c4)),
                                  reinterpret_cast<f32x4*>(Sg1 + (size_t)row * DV + c4));
    }
  }
}

template <int DK, int DV, class Io, bool SG, bool FU>
static void launch_rec_k(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* S0, void* out, float* S_final,
                         const int32_t* cu, unsigned blocks, int T, int H, float scale,
                         const Prologue& pro, hipStream_t stream) {
  hipLaunchKernelGGL((recurrent_fwd_kernel<DK, DV, Io, SG, FU>), dim3(blocks), dim3(256), 0,
                     stream, q, k, v, g, beta, S0, out, S_final, cu, T, H, scale, pro);
}

template <int DK, int DV, class Io>
static hipError_t launch_recurrent_t(const void* q, const void* k, const void* v, const float* g,
                                     const float* beta, const float* S0, void* out,
                                     float* S_final, const int32_t* cu, int n_seq, int T, int H,
                                     float scale, bool sg, const Prologue& pro,
                                     hipStream_t stream) {
  const long blocks = (long)n_seq * H * (DV / 64);
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  const unsigned nb = (unsigned)blocks;
  const bool fu = pro.flags != 0;
  if (sg && fu)
    launch_rec_k<DK, DV, Io, true, true>(q, k, v, g, beta, S0, out, S_final, cu, nb, T, H, scale, pro, stream);
  else if (sg)
    launch_rec_k<DK, DV, Io, true, false>(q, k, v, g, beta, S0, out, S_final, cu, nb, T, H, scale, pro, stream);
  else if (fu)
    launch_rec_k<DK, DV, Io, false, true>(q, k, v, g, beta, S0, out, S_final, cu, nb, T, H, scale, pro, stream);
  else
    launch_rec_k<DK, DV, Io, false, false>(q, k, v, g, beta, S0, out, S_final, cu, nb, T, H, scale, pro, stream);
  return hipGetLastError();
}

hipError_t launch_recurrent(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* S0, void* out, float* S_final,
                            const int32_t* cu, int n_seq, int T, int H, int dk, int dv,
                            float scale, bool bf16, bool scalar_gate, const Prologue& pro,
                            hipStream_t stream) {
#define KDA_REC(DK, DV)                                                                    \
  if (dk == DK && dv == DV)                                                               \
    return bf16 ? launch_recurrent_t<DK, DV, IoBf16>(q, k, v, g, beta, S0, out, S_final, cu, \
                                                     n_seq, T, H, scale, scalar_gate, pro, stream) \
                : launch_recurrent_t<DK, DV, IoF32>(q, k, v, g, beta, S0, out, S_final, cu,  \
                                                    n_seq, T, H, scale, scalar_gate, pro, stream);
  KDA_REC(64, 64)
  KDA_REC(64, 128)
  KDA_REC(128, 64)
  KDA_REC(128, 128)
#undef KDA_REC
  return hipErrorInvalidValue;
}

}  // namespace kda
