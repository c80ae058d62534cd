// kda_api.hip -- the C ABI declared in include/kda.h: validation, then launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "common.h"
#include "kda.h"

namespace kda {
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float* S, void* out, int NH, int H, int dk, int dv,
                         float scale, bool bf16, bool scalar_gate, const Prologue& pro,
                         hipStream_t stream);
hipError_t launch_chunk(const void* q, const void* k, const void* v, const float* g,
                        const float* beta, const float* S0, void* out, float* S_final,
                        const int32_t* cu_seqlens, int n_seq, int T, int H, int dk, int dv,
                        float scale, bool bf16, bool scalar_gate, const Prologue& pro, void* ws,
                        hipStream_t stream);
size_t chunk_split_workspace_bytes(int n_seq, int H, int dk, int dv);
bool chunk_supported(int dk, int dv, bool bf16);
bool chunk_par_selected(int n_seq, int T, int H, int dk, int dv, bool bf16);
bool chunk_par_varlen_selected(int N, int T_total, int H, int dk, int dv, bool bf16);
size_t chunk_par_workspace_bytes(int n_seq, int T, int H);
size_t chunk_par_varlen_workspace_bytes(int N, int T_total, int H);
hipError_t launch_chunk_par(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* S0, void* out, float* S_final,
                            const int32_t* cu, int n_seq, int T, int H, float scale, void* ws,
                            hipStream_t stream);
hipError_t launch_recurrent(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, const float* S0, void* out, float* S_final,
                            const int32_t* cu, int n_seq, int T, int H, int dk, int dv,
                            float scale, bool bf16, bool scalar_gate, const Prologue& pro,
                            hipStream_t stream);
size_t backward_workspace_bytes(int n_seq, size_t rows, int H, int dk, int dv);
hipError_t launch_backward(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const float* S0, const void* dout, const float* dSf,
                           float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                           const int32_t* cu, int n_seq, int T, int H, int d_k, int d_v,
                           float scale, bool bf16, bool scalar_gate, float* ws,
                           hipStream_t stream);
}  // namespace kda

namespace {

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range span(const void* p, size_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}

bool overlap(Range a, Range b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

bool io_ok(int io) { return io == KDA_IO_F32 || io == KDA_IO_BF16; }
size_t io_bytes(int io) { return io == KDA_IO_BF16 ? 2 : 4; }

// Copy S0 (or zeros) into S_final for sequences with no tokens: done by a
// tiny kernel rather than a memset so that the call can sit in a HIP graph.
__global__ void copy_state_kernel(const float* __restrict__ S0, float* __restrict__ Sf, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    Sf[i] = S0 ? S0[i] : 0.f;
}

int launch_status(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool shape_ok(int d) { return d == 64 || d == 128; }

// The vector loads and stores of every kernel assume 16-byte aligned arrays
// (beta and cu_seqlens are read as single words).
// A per-(token, head) gate (scalar_gate) is read as single words too.
int check_align(const void* q, const void* k, const void* v, const float* log_alpha,
                const float* beta, const float* S0, const void* out, const float* S_final,
                const int32_t* cu, bool scalar_gate) {
  const void* a16[] = {q, k, v, S0, out, S_final};
  for (const void* p : a16)
    if (!aligned(p, 16)) return KDA_ERR_ALIGN;
  if (!aligned(log_alpha, scalar_gate ? 4 : 16)) return KDA_ERR_ALIGN;
  if (!aligned(beta, 4) || !aligned(cu, 4)) return KDA_ERR_ALIGN;
  return KDA_OK;
}

// Shared validation of the prefill entry points.  `rows` is the number of
// token rows (B*T or T_total), `n_seq` the number of state slots.
// The input transforms: known flags, A_log present with the gate transform,
// word-aligned parameter arrays that no output overlaps.  Fills `out`.
int check_prologue(const kda_prologue* pro, int H, int d_k, bool sg, kda::Prologue* o,
                   Range r_out, Range r_state) {
  *o = kda::Prologue{0u, nullptr, nullptr};
  if (!pro) return KDA_OK;
  const uint32_t known = KDA_PRO_QK_L2NORM | KDA_PRO_BETA_SIGMOID | KDA_PRO_GATE;
  if (pro->flags & ~known) return KDA_ERR_UNSUPPORTED;
  if (pro->flags & KDA_PRO_GATE) {
    if (!pro->A_log) return KDA_ERR_NULL;
    if (!aligned(pro->A_log, 4) || !aligned(pro->gate_bias, 4)) return KDA_ERR_ALIGN;
    const Range ra = span(pro->A_log, (size_t)H * 4);
    const Range rb = span(pro->gate_bias, pro->gate_bias ? (size_t)H * (sg ? 1 : d_k) * 4 : 0);
    if (overlap(ra, r_out) || overlap(ra, r_state) || overlap(rb, r_out) || overlap(rb, r_state))
      return KDA_ERR_ALIAS;
  }
  // the kernels' bit values equal the header's
  static_assert(KDA_PRO_QK_L2NORM == kda::PRO_L2NORM && KDA_PRO_BETA_SIGMOID == kda::PRO_BETA_SIGMOID &&
                    KDA_PRO_GATE == kda::PRO_GATE,
                "prologue flags");
  o->flags = pro->flags;
  o->A_log = (pro->flags & KDA_PRO_GATE) ? pro->A_log : nullptr;
  o->bias = (pro->flags & KDA_PRO_GATE) ? pro->gate_bias : nullptr;
  return KDA_OK;
}

// Shared validation of the calls over token sequences (prefill and
// recurrent); `supported` is the caller's check of d_k, d_v, chunk and io_dtype.
int check_tokens(const void* q, const void* k, const void* v, const float* log_alpha,
                 const float* beta, const float* S0, void* out, float* S_final,
                 const int32_t* cu, size_t rows, int n_seq, int H, int d_k, int d_v,
                 bool supported, int io_dtype, bool scalar_gate) {
  if (!supported) return KDA_ERR_UNSUPPORTED;
  if (rows > 0 && (!q || !k || !v || !log_alpha || !beta || !out)) return KDA_ERR_NULL;
  const int al = check_align(q, k, v, log_alpha, beta, S0, out, S_final, cu, scalar_gate);
  if (al != KDA_OK) return al;
  const size_t e = io_bytes(io_dtype);
  const size_t state = (size_t)n_seq * H * d_k * d_v * sizeof(float);
  const Range in[] = {span(q, rows * H * d_k * e), span(k, rows * H * d_k * e),
                      span(v, rows * H * d_v * e),
                      span(log_alpha, rows * H * (scalar_gate ? 1 : d_k) * 4),
                      span(beta, rows * H * 4),    span(cu, cu ? (size_t)(n_seq + 1) * 4 : 0)};
  const Range ro = span(out, rows * H * d_v * e);
  const Range rs = span(S_final, S_final ? state : 0);
  const Range r0 = span(S0, S0 ? state : 0);
  for (const Range& r : in) {
    if (overlap(ro, r) || overlap(rs, r)) return KDA_ERR_ALIAS;
  }
  if (overlap(ro, rs) || overlap(ro, r0)) return KDA_ERR_ALIAS;
  if (S_final && S0 && S0 != S_final && overlap(rs, r0)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

int check_prefill(const void* q, const void* k, const void* v, const float* log_alpha,
                  const float* beta, const float* S0, void* out, float* S_final,
                  const int32_t* cu, size_t rows, int n_seq, int H, int d_k, int d_v, int chunk,
                  int io_dtype, bool scalar_gate) {
  const bool ok = io_ok(io_dtype) && chunk == 64 &&
                  kda::chunk_supported(d_k, d_v, io_dtype == KDA_IO_BF16);
  return check_tokens(q, k, v, log_alpha, beta, S0, out, S_final, cu, rows, n_seq, H, d_k, d_v,
                      ok, io_dtype, scalar_gate);
}

int check_recurrent(const void* q, const void* k, const void* v, const float* log_alpha,
                    const float* beta, const float* S0, void* out, float* S_final,
                    const int32_t* cu, size_t rows, int n_seq, int H, int d_k, int d_v,
                    int io_dtype, bool scalar_gate) {
  const bool ok = io_ok(io_dtype) && shape_ok(d_k) && shape_ok(d_v);
  return check_tokens(q, k, v, log_alpha, beta, S0, out, S_final, cu, rows, n_seq, H, d_k, d_v,
                      ok, io_dtype, scalar_gate);
}

}  // namespace

namespace {

// One implementation per operation; cu_seqlens NULL means the batched
// layout (n_seq sequences of T tokens), otherwise the packed one (T = T_total).
// Workspace of the plain batched KDA prefill: the chunk-parallel schedule's
// per-chunk factors when that schedule is selected for these sizes, else none.
// The chunk-parallel schedule's factors for the shapes that take it (plain
// KDA calls of few long chains), else the balanced schedule's plan and
// hand-over states.
size_t chunk_ws_bytes(int B, int T, int H, int d_k, int d_v, int chunk, int io_dtype) {
  if (B <= 0 || T < 0 || H <= 0 || chunk != 64 || !io_ok(io_dtype)) return 0;
  const bool bf16 = io_dtype == KDA_IO_BF16;
  if (!kda::chunk_supported(d_k, d_v, bf16)) return 0;
  if (kda::chunk_par_selected(B, T, H, d_k, d_v, bf16)) return kda::chunk_par_workspace_bytes(B, T, H);
  return kda::chunk_split_workspace_bytes(B, H, d_k, d_v);
}

int chunk_impl(const void* q, const void* k, const void* v, const float* log_alpha,
               const float* beta, const float* S0, void* out, float* S_final,
               const int32_t* cu_seqlens, bool packed, int n_seq, int T, int H, int d_k, int d_v,
               float scale, int chunk, int io_dtype, bool sg, const kda_prologue* pro,
               void* stream, void* workspace = nullptr, size_t workspace_bytes = 0) {
  if (n_seq < 0 || T < 0 || H <= 0) return KDA_ERR_DIM;
  if (packed && !cu_seqlens) return KDA_ERR_NULL;
  const size_t rows = packed ? (size_t)T : (size_t)n_seq * T;
  if (rows > 0x7fffffffu) return KDA_ERR_DIM;   // token rows are 32-bit in the kernels
  int st = check_prefill(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, rows, n_seq, H,
                         d_k, d_v, chunk, io_dtype, sg);
  if (st != KDA_OK) return st;
  kda::Prologue pr;
  const size_t state = (size_t)n_seq * H * d_k * d_v * 4;
  st = check_prologue(pro, H, d_k, sg, &pr, span(out, rows * H * d_v * io_bytes(io_dtype)),
                      span(S_final, S_final ? state : 0));
  if (st != KDA_OK) return st;
  // the chunk-parallel schedule (plain KDA calls of few long chains; packed
  // calls take it when given a workspace, batched ones need one)
  const bool bf16 = io_dtype == KDA_IO_BF16;
  const bool par = !sg && pr.flags == 0 &&
                   (packed ? workspace && kda::chunk_par_varlen_selected(n_seq, T, H, d_k, d_v, bf16)
                           : kda::chunk_par_selected(n_seq, T, H, d_k, d_v, bf16));
  if (par) {
    const size_t need = packed ? kda::chunk_par_varlen_workspace_bytes(n_seq, T, H)
                               : kda::chunk_par_workspace_bytes(n_seq, T, H);
    if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KDA_ERR_ALIGN;
    const size_t e = io_bytes(io_dtype);
    const Range rw = span(workspace, need);
    const Range others[] = {span(q, rows * H * d_k * e), span(k, rows * H * d_k * e),
                            span(v, rows * H * d_v * e), span(log_alpha, rows * H * d_k * 4),
                            span(beta, rows * H * 4), span(S0, S0 ? state : 0),
                            span(out, rows * H * d_v * e), span(S_final, S_final ? state : 0),
                            span(cu_seqlens, cu_seqlens ? ((size_t)n_seq + 1) * 4 : 0)};
    for (const Range& r : others)
      if (overlap(rw, r)) return KDA_ERR_ALIAS;
  }
  // otherwise a workspace enables the balanced schedule (taken when there are
  // more chains than resident workgroups)
  void* split_ws = nullptr;
  if (!par && workspace) {
    const size_t need = kda::chunk_split_workspace_bytes(n_seq, H, d_k, d_v);
    if (workspace_bytes < need) return KDA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return KDA_ERR_ALIGN;
    const size_t e = io_bytes(io_dtype);
    const Range rw = span(workspace, need);
    const Range others[] = {span(q, rows * H * d_k * e), span(k, rows * H * d_k * e),
                            span(v, rows * H * d_v * e),
                            span(log_alpha, rows * H * (sg ? 1 : d_k) * 4),
                            span(beta, rows * H * 4), span(S0, S0 ? state : 0),
                            span(out, rows * H * d_v * e), span(S_final, S_final ? state : 0),
                            span(cu_seqlens, cu_seqlens ? ((size_t)n_seq + 1) * 4 : 0)};
    for (const Range& r : others)
      if (overlap(rw, r)) return KDA_ERR_ALIAS;
    split_ws = workspace;
  }
  if (n_seq == 0) return KDA_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (par)
    return launch_status(kda::launch_chunk_par(q, k, v, log_alpha, beta, S0, out, S_final,
                                               packed ? cu_seqlens : nullptr, n_seq, T, H, scale,
                                               workspace, s));
  if (!packed && T == 0) {
    if (!S_final || S0 == S_final) return KDA_OK;
    hipLaunchKernelGGL(copy_state_kernel, dim3(1024), dim3(256), 0, s, S0, S_final, state / 4);
    return launch_status(hipGetLastError());
  }
  return launch_status(kda::launch_chunk(q, k, v, log_alpha, beta, S0, out, S_final,
                                         packed ? cu_seqlens : nullptr, n_seq, T, H, d_k, d_v,
                                         scale, io_dtype == KDA_IO_BF16, sg, pr, split_ws, s));
}

int decode_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                const float* beta, float* S_inout, void* out, int N, int H, int d_k, int d_v,
                float scale, int io_dtype, bool sg, const kda_prologue* pro, void* stream) {
  if (N < 0 || H <= 0) return KDA_ERR_DIM;
  if (!io_ok(io_dtype)) return KDA_ERR_UNSUPPORTED;
  if (!(shape_ok(d_k) && shape_ok(d_v))) return KDA_ERR_UNSUPPORTED;
  if (N == 0) return KDA_OK;
  if (!q || !k || !v || !log_alpha || !beta || !S_inout || !out) return KDA_ERR_NULL;
  const int al = check_align(q, k, v, log_alpha, beta, S_inout, out, nullptr, nullptr, sg);
  if (al != KDA_OK) return al;
  const size_t e = io_bytes(io_dtype);
  const size_t heads = (size_t)N * H;
  const Range in[] = {span(q, heads * d_k * e), span(k, heads * d_k * e), span(v, heads * d_v * e),
                      span(log_alpha, heads * (sg ? 1 : d_k) * 4), span(beta, heads * 4)};
  const Range ro = span(out, heads * d_v * e);
  const Range rs = span(S_inout, heads * d_k * d_v * 4);
  for (const Range& r : in) {
    if (overlap(ro, r) || overlap(rs, r)) return KDA_ERR_ALIAS;
  }
  if (overlap(ro, rs)) return KDA_ERR_ALIAS;
  kda::Prologue pr;
  const int sp = check_prologue(pro, H, d_k, sg, &pr, ro, rs);
  if (sp != KDA_OK) return sp;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return launch_status(kda::launch_decode(q, k, v, log_alpha, beta, S_inout, out, (int)heads, H,
                                          d_k, d_v, scale, io_dtype == KDA_IO_BF16, sg, pr, s));
}

int recurrent_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                   const float* beta, const float* S0, void* out, float* S_final,
                   const int32_t* cu_seqlens, bool packed, int n_seq, int T, int H, int d_k,
                   int d_v, float scale, int io_dtype, bool sg, const kda_prologue* pro,
                   void* stream) {
  if (n_seq < 0 || T < 0 || H <= 0) return KDA_ERR_DIM;
  if (packed && !cu_seqlens) return KDA_ERR_NULL;
  const size_t rows = packed ? (size_t)T : (size_t)n_seq * T;
  if (rows > 0x7fffffffu) return KDA_ERR_DIM;   // token indices are 32-bit in the kernel
  int st = check_recurrent(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, rows, n_seq,
                           H, d_k, d_v, io_dtype, sg);
  if (st != KDA_OK) return st;
  kda::Prologue pr;
  const size_t state = (size_t)n_seq * H * d_k * d_v * 4;
  st = check_prologue(pro, H, d_k, sg, &pr, span(out, rows * H * d_v * io_bytes(io_dtype)),
                      span(S_final, S_final ? state : 0));
  if (st != KDA_OK) return st;
  if (n_seq == 0) return KDA_OK;
  if (!packed && T == 0 && (!S_final || S0 == S_final)) return KDA_OK;
  // (T == 0 with a separate S_final: the kernel copies S0, or zeros, through)
  return launch_status(kda::launch_recurrent(q, k, v, log_alpha, beta, S0, out, S_final,
                                             packed ? cu_seqlens : nullptr, n_seq, T, H, d_k, d_v,
                                             scale, io_dtype == KDA_IO_BF16, sg, pr,
                                             reinterpret_cast<hipStream_t>(stream)));
}

int backward_impl(const void* q, const void* k, const void* v, const float* log_alpha,
                  const float* beta, const float* S0, const void* d_out, const float* dS_final,
                  float* dq, float* dk, float* dv, float* dg, float* dbeta, float* dS0,
                  const int32_t* cu_seqlens, int n_seq, int T, int H, int d_k, int d_v,
                  float scale, int io_dtype, bool sg, void* workspace, size_t workspace_bytes,
                  void* stream, bool check_only = false) {
  // check_only: validate everything except the workspace and enqueue nothing
  if (n_seq < 0 || T < 0 || H <= 0) return KDA_ERR_DIM;
  if (!io_ok(io_dtype) || !shape_ok(d_k) || !shape_ok(d_v)) return KDA_ERR_UNSUPPORTED;
  const bool packed = cu_seqlens != nullptr;
  const size_t rows = packed ? (size_t)T : (size_t)n_seq * T;
  if (rows > 0x7fffffffu) return KDA_ERR_DIM;
  if ((size_t)n_seq * H > 0x7fffffffu) return KDA_ERR_DIM;   // one workgroup per chain
  if (rows > 0 && (!q || !k || !v || !log_alpha || !beta || !d_out || !dq || !dk || !dv || !dg ||
                   !dbeta))
    return KDA_ERR_NULL;
  const void* a16[] = {q, k, v, S0, d_out, dS_final, dq, dk, dv, dS0, workspace};
  for (const void* p : a16)
    if (!aligned(p, 16)) return KDA_ERR_ALIGN;
  const void* a4[] = {log_alpha, beta, cu_seqlens, dg, dbeta};
  for (const void* p : a4)
    if (!aligned(p, 4)) return KDA_ERR_ALIGN;
  const size_t need = kda::backward_workspace_bytes(n_seq, rows, H, d_k, d_v);
  if (!check_only && n_seq > 0 && (!workspace || workspace_bytes < need)) return KDA_ERR_WORKSPACE;
  const size_t e = io_bytes(io_dtype);
  const size_t state = (size_t)n_seq * H * d_k * d_v * 4;
  const size_t gk = rows * H * (sg ? 1 : d_k) * 4;
  const Range in[] = {span(q, rows * H * d_k * e),     span(k, rows * H * d_k * e),
                      span(v, rows * H * d_v * e),     span(log_alpha, gk),
                      span(beta, rows * H * 4),        span(S0, S0 ? state : 0),
                      span(d_out, rows * H * d_v * e), span(dS_final, dS_final ? state : 0),
                      span(cu_seqlens, packed ? (size_t)(n_seq + 1) * 4 : 0)};
  const Range outs[] = {span(dq, rows * H * d_k * 4), span(dk, rows * H * d_k * 4),
                        span(dv, rows * H * d_v * 4), span(dg, gk),
                        span(dbeta, rows * H * 4),    span(dS0, dS0 ? state : 0),
                        span(workspace, n_seq > 0 && !check_only ? need : 0)};
  for (size_t i = 0; i < sizeof(outs) / sizeof(outs[0]); ++i) {
    for (const Range& r : in)
      if (overlap(outs[i], r)) return KDA_ERR_ALIAS;
    for (size_t j = i + 1; j < sizeof(outs) / sizeof(outs[0]); ++j)
      if (overlap(outs[i], outs[j])) return KDA_ERR_ALIAS;
  }
  if (n_seq == 0 || check_only) return KDA_OK;
  return launch_status(kda::launch_backward(q, k, v, log_alpha, beta, S0, d_out, dS_final, dq, dk,
                                            dv, dg, dbeta, dS0, cu_seqlens, n_seq, T, H, d_k, d_v,
                                            scale, io_dtype == KDA_IO_BF16, sg,
                                            reinterpret_cast<float*>(workspace),
                                            reinterpret_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------------ static scratch
// The allocation-free backward (kda_backward_noalloc) keeps its workspace in
// this array instead of caller memory.  Each device that loads the library
// holds its own copy, at its own address, until the process ends.  In host
// code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress with that device current, once per device, and is the
// only form in which the array is handed to a kernel.
constexpr size_t kScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first call on that device).
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KDA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_version(void) { return 100; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_DIM: return "KDA_ERR_DIM: a size is negative or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: d_k, d_v, chunk or io_dtype not supported";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: a HIP launch failed";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: an array is not 16-byte aligned";
    case KDA_ERR_SCRATCH:
      return "KDA_ERR_SCRATCH: the problem needs more scratch than the static buffer holds";
    default: return "unknown KDA status";
  }
}

size_t kda_chunk_fwd_workspace_size(int B, int T, int H, int d_k, int d_v, int chunk,
                                    int io_dtype) {
  return chunk_ws_bytes(B, T, H, d_k, d_v, chunk, io_dtype);
}

size_t kda_chunk_fwd_varlen_workspace_size(int N, int T_total, int H, int d_k, int d_v,
                                           int chunk, int io_dtype) {
  const bool bf16 = io_dtype == KDA_IO_BF16;
  if (N <= 0 || T_total < 0 || H <= 0 || chunk != 64 || !io_ok(io_dtype) ||
      !kda::chunk_supported(d_k, d_v, bf16))
    return 0;
  if (kda::chunk_par_varlen_selected(N, T_total, H, d_k, d_v, bf16))
    return kda::chunk_par_varlen_workspace_bytes(N, T_total, H);
  return kda::chunk_split_workspace_bytes(N, H, d_k, d_v);
}

int kda_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                  const float* beta, const float* S0, void* out, float* S_final, int B, int T,
                  int H, int d_k, int d_v, float scale, int chunk, int io_dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
  return chunk_impl(q, k, v, log_alpha, beta, S0, out, S_final, nullptr, false, B, T, H, d_k, d_v,
                    scale, chunk, io_dtype, false, nullptr, stream, workspace, workspace_bytes);
}

int kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* S0, void* out, float* S_final,
                         const int32_t* cu_seqlens, int N, int T_total, int H, int d_k, int d_v,
                         float scale, int chunk, int io_dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return chunk_impl(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, true, N, T_total, H,
                    d_k, d_v, scale, chunk, io_dtype, false, nullptr, stream,
                    workspace, workspace_bytes);
}

int kda_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                    const float* beta, float* S_inout, void* out, int N, int H, int d_k, int d_v,
                    float scale, int io_dtype, void* stream) {
  return decode_impl(q, k, v, log_alpha, beta, S_inout, out, N, H, d_k, d_v, scale, io_dtype,
                     false, nullptr, stream);
}

int kda_recurrent_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                      const float* beta, const float* S0, void* out, float* S_final, int B, int T,
                      int H, int d_k, int d_v, float scale, int io_dtype, void* stream) {
  return recurrent_impl(q, k, v, log_alpha, beta, S0, out, S_final, nullptr, false, B, T, H, d_k,
                        d_v, scale, io_dtype, false, nullptr, stream);
}

int kda_recurrent_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const float* S0, void* out, float* S_final,
                             const int32_t* cu_seqlens, int N, int T_total, int H, int d_k,
                             int d_v, float scale, int io_dtype, void* stream) {
  return recurrent_impl(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, true, N, T_total,
                        H, d_k, d_v, scale, io_dtype, false, nullptr, stream);
}

int kda_gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                      const float* beta, const float* S0, void* out, float* S_final, int B, int T,
                      int H, int d_k, int d_v, float scale, int chunk, int io_dtype,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_impl(q, k, v, log_alpha, beta, S0, out, S_final, nullptr, false, B, T, H, d_k, d_v,
                    scale, chunk, io_dtype, true, nullptr, stream, workspace, workspace_bytes);
}

int kda_gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const float* log_alpha,
                             const float* beta, const float* S0, void* out, float* S_final,
                             const int32_t* cu_seqlens, int N, int T_total, int H, int d_k,
                             int d_v, float scale, int chunk, int io_dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return chunk_impl(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, true, N, T_total, H,
                    d_k, d_v, scale, chunk, io_dtype, true, nullptr, stream,
                    workspace, workspace_bytes);
}

int kda_gdn_decode_step(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, float* S_inout, void* out, int N, int H, int d_k,
                        int d_v, float scale, int io_dtype, void* stream) {
  return decode_impl(q, k, v, log_alpha, beta, S_inout, out, N, H, d_k, d_v, scale, io_dtype,
                     true, nullptr, stream);
}

int kda_gdn_recurrent_fwd(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, const float* S0, void* out, float* S_final, int B,
                          int T, int H, int d_k, int d_v, float scale, int io_dtype,
                          void* stream) {
  return recurrent_impl(q, k, v, log_alpha, beta, S0, out, S_final, nullptr, false, B, T, H, d_k,
                        d_v, scale, io_dtype, true, nullptr, stream);
}

int kda_gdn_recurrent_fwd_varlen(const void* q, const void* k, const void* v,
                                 const float* log_alpha, const float* beta, const float* S0,
                                 void* out, float* S_final, const int32_t* cu_seqlens, int N,
                                 int T_total, int H, int d_k, int d_v, float scale, int io_dtype,
                                 void* stream) {
  return recurrent_impl(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, true, N, T_total,
                        H, d_k, d_v, scale, io_dtype, true, nullptr, stream);
}

int kda_chunk_fwd_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                        const float* beta, const float* S0, void* out, float* S_final,
                        const int32_t* cu_seqlens, int N, int T, int H, int d_k, int d_v,
                        float scale, int chunk, int io_dtype, int per_head_gate,
                        const kda_prologue* pro, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (per_head_gate != 0 && per_head_gate != 1) return KDA_ERR_UNSUPPORTED;
  return chunk_impl(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens, cu_seqlens != nullptr,
                    N, T, H, d_k, d_v, scale, chunk, io_dtype, per_head_gate == 1, pro, stream,
                    workspace, workspace_bytes);
}

int kda_recurrent_fwd_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                            const float* beta, const float* S0, void* out, float* S_final,
                            const int32_t* cu_seqlens, int N, int T, int H, int d_k, int d_v,
                            float scale, int io_dtype, int per_head_gate,
                            const kda_prologue* pro, void* stream) {
  if (per_head_gate != 0 && per_head_gate != 1) return KDA_ERR_UNSUPPORTED;
  return recurrent_impl(q, k, v, log_alpha, beta, S0, out, S_final, cu_seqlens,
                        cu_seqlens != nullptr, N, T, H, d_k, d_v, scale, io_dtype,
                        per_head_gate == 1, pro, stream);
}

int kda_decode_step_fused(const void* q, const void* k, const void* v, const float* log_alpha,
                          const float* beta, float* S_inout, void* out, int N, int H, int d_k,
                          int d_v, float scale, int io_dtype, int per_head_gate,
                          const kda_prologue* pro, void* stream) {
  if (per_head_gate != 0 && per_head_gate != 1) return KDA_ERR_UNSUPPORTED;
  return decode_impl(q, k, v, log_alpha, beta, S_inout, out, N, H, d_k, d_v, scale, io_dtype,
                     per_head_gate == 1, pro, stream);
}

size_t kda_backward_workspace_size(int N, int T, int H, int d_k, int d_v, int packed) {
  if (N < 0 || T < 0 || H <= 0 || !shape_ok(d_k) || !shape_ok(d_v)) return 0;
  const size_t rows = packed ? (size_t)T : (size_t)N * T;
  return kda::backward_workspace_bytes(N, rows, H, d_k, d_v);
}

int kda_backward(const void* q, const void* k, const void* v, const float* log_alpha,
                 const float* beta, const float* S0, const void* d_out, const float* dS_final,
                 float* dq, float* dk, float* dv, float* dlog_alpha, float* dbeta, float* dS0,
                 const int32_t* cu_seqlens, int N, int T, int H, int d_k, int d_v, float scale,
                 int io_dtype, int per_head_gate, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (per_head_gate != 0 && per_head_gate != 1) return KDA_ERR_UNSUPPORTED;
  return backward_impl(q, k, v, log_alpha, beta, S0, d_out, dS_final, dq, dk, dv, dlog_alpha,
                       dbeta, dS0, cu_seqlens, N, T, H, d_k, d_v, scale, io_dtype,
                       per_head_gate == 1, workspace, workspace_bytes, stream);
}

size_t kda_noalloc_scratch_bytes(void) { return kScratchBytes; }

int kda_backward_noalloc(const void* q, const void* k, const void* v, const float* log_alpha,
                         const float* beta, const float* S0, const void* d_out,
                         const float* dS_final, float* dq, float* dk, float* dv,
                         float* dlog_alpha, float* dbeta, float* dS0,
                         const int32_t* cu_seqlens, int N, int T, int H, int d_k, int d_v,
                         float scale, int io_dtype, int per_head_gate, void* stream) {
  if (per_head_gate != 0 && per_head_gate != 1) return KDA_ERR_UNSUPPORTED;
  // every argument first, with nothing enqueued and no HIP call
  int st = backward_impl(q, k, v, log_alpha, beta, S0, d_out, dS_final, dq, dk, dv, dlog_alpha,
                         dbeta, dS0, cu_seqlens, N, T, H, d_k, d_v, scale, io_dtype,
                         per_head_gate == 1, nullptr, 0, stream, /*check_only=*/true);
  if (st != KDA_OK) return st;
  const size_t rows = cu_seqlens ? (size_t)T : (size_t)N * T;
  if (kda::backward_workspace_bytes(N, rows, H, d_k, d_v) > kScratchBytes) return KDA_ERR_SCRATCH;
  if (N == 0) return KDA_OK;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != KDA_OK) return st;
  // Every word of the workspace the kernel reads, it wrote earlier in the
  // same call (checkpoints and v - p), so nothing needs clearing.
  return backward_impl(q, k, v, log_alpha, beta, S0, d_out, dS_final, dq, dk, dv, dlog_alpha,
                       dbeta, dS0, cu_seqlens, N, T, H, d_k, d_v, scale, io_dtype,
                       per_head_gate == 1, ws, kScratchBytes, stream);
}

}  // extern "C"
